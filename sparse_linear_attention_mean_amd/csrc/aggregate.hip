// Marginal aggregation as a bit-masked GEMM on bf16 MFMA (gfx950).
//
// The linear branch of SLA ("SLA: Beyond Sparsity in Diffusion Transformers
// via Fine-Tunable Sparse-Linear Attention", method section, step 3 -- linear
// attention over the marginal weights) needs, per query block i, the sums
//   H_i = sum_{j marginal for i} h_j,   Z_i = sum_{j marginal for i} z_j.
// Summing per row would gather hundreds of d x d states per query block; here
// all rows of a head are produced at once as C = M0 * S, where M0 is the 0/1
// marginal matrix (exact in bf16) and S holds one state row per key block.
// The same kernel serves the backward with the transposed marginal matrix
// (dh_j = sum_{i : j marginal for i} dH_i).
//
// Operands: S in the K-tiled layout states[bh][j / 4][n][j % 4] (bf16), so
// that two 8-byte reads give a lane the 8 consecutive key blocks an MFMA A
// operand needs; M0 as 32-bit words of marginal bits, stored word-major
// (word w of every row contiguous), expanded to bf16 through a 256-entry LDS
// table.  C^T[n][i] = sum_j S[j][n] M0[i][j] is
// computed with v_mfma_f32_16x16x32_bf16, fp32 accumulation.  Columns
// n < D*D are stored as bf16 (H_i transposed, element (c, a) at c*D + a);
// the 2*D columns after them (z split into two bf16 parts) as fp32.
#include "sla_device.h"
#include "sla_internal.h"

namespace sla {

constexpr int kAggNTile = 64;    // state columns per workgroup
constexpr int kAggIWave = 128;   // query rows per wave
constexpr int kAggIChunk = 512;  // query rows per workgroup (4 waves)
constexpr int kAggKChunk = 128;  // key blocks of the state strip staged in LDS per chunk
// LDS strip: pairs of 4-block planes, 2 x 64 columns x 4 blocks (1 KB, one
// copy instruction) plus 128 bytes of padding, so the four lane groups of an
// A-operand read (planes 2 g apart) fall on different banks
constexpr int kAggPair = 2 * kAggNTile * 4 + 64;   // bf16 elements per plane pair

// One workgroup owns a 64-column strip of S and 512 rows of C.  The strip is
// shared by the four waves (each owns 128 rows), so it is copied into LDS with
// asynchronous global->LDS loads instead of being fetched by every wave, in
// chunks of 128 key blocks (18 KB) into two buffers: the next chunk's copies
// are in flight while the current chunk is multiplied (the buffers are
// separate arrays named statically, so the compiler does not hold the LDS
// reads back for the copies in flight).  The marginal words stream from
// global memory (they are small and stay in L2) two k-steps ahead, 32
// contiguous bytes per lane and k-step.
__global__ __launch_bounds__(256, 2) void aggregate_kernel(const uint32_t* __restrict__ bits,
                                                          const uint16_t* __restrict__ states,
                                                          uint16_t* __restrict__ hout,
                                                          float* __restrict__ zout, int T, int Tp,
                                                          int NB, int DD, int ntiles,
                                                          int ichunks) {
  __shared__ u32x4 table[256];
  __shared__ __attribute__((aligned(16))) uint16_t strip0[kAggKChunk / 8 * kAggPair];
  __shared__ __attribute__((aligned(16))) uint16_t strip1[kAggKChunk / 8 * kAggPair];
  // the chunk's marginal words: word k of rows ib .. ib + 511 at [k][row - ib]
  __shared__ __attribute__((aligned(16))) uint32_t wsl0[kAggKChunk / 32 * kAggIChunk];
  __shared__ __attribute__((aligned(16))) uint32_t wsl1[kAggKChunk / 32 * kAggIChunk];
  const int tid = threadIdx.x;
  {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = ((tid >> (2 * p)) & 1 ? 0x3F80u : 0u) | ((tid >> (2 * p + 1)) & 1 ? 0x3F800000u : 0u);
    table[tid] = u32x4{w[0], w[1], w[2], w[3]};
  }

  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = wg % ntiles;
  const int rest = wg / ntiles;
  const int ic = rest % ichunks;
  const long long bh = rest / ichunks;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = nt * kAggNTile;
  const int i0 = ic * kAggIChunk + wave * kAggIWave;
  // Tile q, column r16 of this wave is query row i0 + 8 r16 + q: a lane's eight
  // rows are consecutive, so its marginal words for one k-step are 32 contiguous
  // bytes of the word-major bit matrix.
  const int rbase = i0 + 8 * r16;
  const bool rows_ok = rbase < Tp;   // lanes past the padded row count compute, never store

  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* sbase = states + static_cast<size_t>(bh) * Tp * NB;
  const int ksteps = Tp / 32;
  const int ib = ic * kAggIChunk;
  // bits of this workgroup's rows, bounded at the padded row count (rows past
  // it read as zero)
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(bits + static_cast<size_t>(bh) * ksteps * Tp, static_cast<uint32_t>(ksteps) * Tp * 4u);
  // one k-step (32 key blocks): A = S^T tile from the staged strip, B = bits -> bf16
  auto step = [&](const uint16_t* strip, const uint32_t* wsl, int kl) __attribute__((always_inline)) {
    const uint32_t* wr = wsl + kl * kAggIChunk + (rbase - ib);   // rows rbase .. rbase + 7
    const u32x4 wlo = *reinterpret_cast<const u32x4*>(wr);
    const u32x4 whi = *reinterpret_cast<const u32x4*>(wr + 4);
    bf16x8 a[4], b[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // planes 8 kl + 2 g and 8 kl + 2 g + 1 = pair 4 kl + g, halves 0 and 1
      const uint16_t* pr = strip + (4 * kl + g) * kAggPair + (16 * m + r16) * 4;
      a[m] = as_bf16x8(ld8(pr), ld8(pr + kAggNTile * 4));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      b[q] = as_bf16x8(table[((q < 4 ? wlo[q & 3] : whi[q & 3]) >> (8 * g)) & 0xffu]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[m][q] = mfma16(a[m], b[q], acc[m][q]);
  };

  // chunk c of the strip (key blocks 128 c ..) into dst: plane pair gi goes
  // to dst + gi * kAggPair, lanes 0-31 plane 2 gi, lanes 32-63 plane 2 gi + 1
  const int nch = (Tp + kAggKChunk - 1) / kAggKChunk;
  // ... and its marginal words: k-step k, 512 rows = 2 KB, one copy of
  // 1 KB per half (waves 0-3 take the k-steps in turn)
  auto copy_chunk = [&](int c, uint16_t* dst, uint32_t* wdst) __attribute__((always_inline)) {
    const int kc0 = c * kAggKChunk;
    const int kn = Tp - kc0 < kAggKChunk ? Tp - kc0 : kAggKChunk;   // multiple of 32
    for (int gi = wave; gi < kn / 8; gi += 4)
      gl_to_lds16(sbase + (static_cast<size_t>(kc0 / 4 + 2 * gi + (lane >> 5)) * NB + n0 +
                           2 * (lane & 31)) * 4,
                  dst + gi * kAggPair);
    for (int h = wave; h < kn / 32 * 2; h += 4) {   // half h: k-step h / 2, rows 256 (h % 2) ..
      const int kk = kc0 / 32 + h / 2;
      const uint32_t off = (static_cast<uint32_t>(kk) * Tp + ib + 256 * (h & 1) + 4 * lane) * 4u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          brs, (__attribute__((address_space(3))) void*)(wdst + (h / 2) * kAggIChunk + 256 * (h & 1)),
          16, off, 0, 0, 0);
    }
  };
  auto chunk = [&](int c, const uint16_t* strip, const uint32_t* wsl) __attribute__((always_inline)) {
    const int kc0 = c * kAggKChunk;
    const int ks = (Tp - kc0 < kAggKChunk ? Tp - kc0 : kAggKChunk) / 32;
    for (int kl = 0; kl < ks; ++kl) step(strip, wsl, kl);
  };

  copy_chunk(0, strip0, wsl0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();   // table ready, chunk 0 in place
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) copy_chunk(c + 1, strip1, wsl1);
    chunk(c, strip0, wsl0);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies into strip1 have landed
    __syncthreads();                 // strip0 consumed, strip1 complete
    if (c + 1 < nch) {
      if (c + 2 < nch) copy_chunk(c + 2, strip0, wsl0);
      chunk(c + 1, strip1, wsl1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // acc[m][q][s] = C^T[n0 + 16 m + 4 g + s][rbase + q]
  if (n0 < DD) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = rbase + q;
      if (!rows_ok || i >= T) continue;
      uint16_t* dst = hout + (static_cast<size_t>(bh) * T + i) * DD + n0 + 4 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        st8(dst + 16 * m, u32x2{pack_bf16x2(acc[m][q][0], acc[m][q][1]),
                                pack_bf16x2(acc[m][q][2], acc[m][q][3])});
      }
    }
  } else {
    const int zw = NB - DD;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = rbase + q;
      if (!rows_ok || i >= T) continue;
      float* dst = zout + (static_cast<size_t>(bh) * T + i) * zw + (n0 - DD) + 4 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<float4*>(dst + 16 * m) =
            make_float4(acc[m][q][0], acc[m][q][1], acc[m][q][2], acc[m][q][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// state_total: the global linear branch (every key block in every row) needs
// one sum per head instead of one per query block, H = sum_j h_j and
// Z = sum_j z_j: a column sum of the state matrix, fp32 in block order, one
// thread per state entry (8-byte loads of the 4-block planes, consecutive
// threads on consecutive entries).  Written like the aggregation output, to
// query-block slot 0 of the head.  Blocks j >= T hold zero states.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void state_total_kernel(const uint16_t* __restrict__ states,
                                                          uint16_t* __restrict__ hout,
                                                          float* __restrict__ zout, int T, int Tp,
                                                          int NB, int DD) {
  const long long bh = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= NB) return;
  const uint16_t* src = states + static_cast<size_t>(bh) * Tp * NB + static_cast<size_t>(n) * 4;
  float acc = 0.f;
  for (int p = 0; p < Tp / 4; p += 8) {   // Tp / 4 is a multiple of 8
    u32x2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld8(src + static_cast<size_t>(p + u) * NB * 4);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += bf16_to_f32(u4_half(v[u], e));
  }
  if (n < DD)
    hout[static_cast<size_t>(bh) * T * DD + n] = f32_to_bf16(acc);
  else
    zout[static_cast<size_t>(bh) * T * (NB - DD) + (n - DD)] = acc;
}

hipError_t launch_state_total(const Dims& d, const uint16_t* states, uint16_t* hout, float* zout,
                              hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((d.NB + 255) / 256), static_cast<unsigned>(d.BH()));
  hipLaunchKernelGGL(state_total_kernel, grid, dim3(256), 0, s, states, hout, zout, d.T, d.Tp, d.NB,
                     d.D * d.D);
  return hipGetLastError();
}

hipError_t launch_aggregate(const Dims& d, const uint32_t* bits, const uint16_t* states,
                            uint16_t* hout, float* zout, hipStream_t s) {
  const int ntiles = d.NB / kAggNTile;
  const int ichunks = (d.Tp + kAggIChunk - 1) / kAggIChunk;
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(ntiles) * ichunks * d.BH()));
  hipLaunchKernelGGL(aggregate_kernel, grid, dim3(256), 0, s, bits, states, hout, zout, d.T, d.Tp,
                     d.NB, d.D * d.D, ntiles, ichunks);
  return hipGetLastError();
}

}  // namespace sla
