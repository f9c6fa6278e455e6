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
// Operands: S in the K-tiled layout states[bh][j / 8][n][j % 8] (bf16), so
// that one 16-byte load gives a lane the 8 consecutive key blocks an MFMA A
// operand needs; M0 as 32-bit words of marginal bits per row, expanded to
// bf16 through a 256-entry LDS table.  C^T[n][i] = sum_j S[j][n] M0[i][j] is
// computed with v_mfma_f32_16x16x32_bf16, fp32 accumulation.  Columns
// n < D*D are stored as bf16 (H_i transposed, element (c, a) at c*D + a);
// the 2*D columns after them (z split into two bf16 parts) as fp32.
#include "sla_device.h"
#include "sla_internal.h"

namespace sla {

constexpr int kAggNTile = 64;    // state columns per workgroup
constexpr int kAggIWave = 128;   // query rows per wave
constexpr int kAggIChunk = 512;  // query rows per workgroup (4 waves)

__global__ __launch_bounds__(256, 2) void aggregate_kernel(const uint32_t* __restrict__ bits,
                                                          const uint16_t* __restrict__ states,
                                                          uint16_t* __restrict__ hout,
                                                          float* __restrict__ zout, int T, int Tp,
                                                          int NB, int DD, int ntiles,
                                                          int ichunks) {
  __shared__ u32x4 table[256];
  const int tid = threadIdx.x;
  {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = ((tid >> (2 * p)) & 1 ? 0x3F80u : 0u) | ((tid >> (2 * p + 1)) & 1 ? 0x3F800000u : 0u);
    table[tid] = u32x4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();

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
  if (i0 >= Tp) return;
  const int words = Tp / 32;
  int nval = (Tp - i0) / 16;     // valid 16-row tiles of this wave
  if (nval > 8) nval = 8;

  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A operand (states) through a buffer resource of this head: lane part of the
  // byte offset in a VGPR, the k step and column tile in the SGPR offset.
  const uint32_t sbytes = static_cast<uint32_t>(Tp / 8) * NB * 16u;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(states + static_cast<size_t>(bh) * (Tp / 8) * NB * 8, sbytes);
  const uint32_t voff = (static_cast<uint32_t>(g) * NB + r16) * 16u;
  const uint32_t* bbase = bits + static_cast<size_t>(bh) * Tp * words;
  const int ksteps = Tp / 32;
  // marginal-bit words of this lane's rows; rows past the wave's valid tiles read nothing
  const uint32_t* brow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) brow[q] = bbase + static_cast<size_t>(i0 + 16 * q + r16) * words;

  u32x4 an[4];
  uint32_t wn[8];
  auto fetch = [&](int kk) {
    const uint32_t soff = (static_cast<uint32_t>(4 * kk) * NB + n0) * 16u;
#pragma unroll
    for (int m = 0; m < 4; ++m) an[m] = buf_ld16(srs, voff, soff + 256u * m);
#pragma unroll
    for (int q = 0; q < 8; ++q) wn[q] = q < nval ? brow[q][kk] : 0u;
  };
  fetch(0);
  for (int kk = 0; kk < ksteps; ++kk) {
    bf16x8 a[4], b[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = as_bf16x8(an[m]);
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q] = as_bf16x8(table[(wn[q] >> (8 * g)) & 0xffu]);
    if (kk + 1 < ksteps) fetch(kk + 1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[m][q] = mfma16(a[m], b[q], acc[m][q]);
  }

  // acc[m][q][s] = C^T[n0 + 16 m + 4 g + s][i0 + 16 q + r16]
  if (n0 < DD) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = i0 + 16 * q + r16;
      if (q >= nval || i >= T) continue;
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
      const int i = i0 + 16 * q + r16;
      if (q >= nval || i >= T) continue;
      float* dst = zout + (static_cast<size_t>(bh) * T + i) * zw + (n0 - DD) + 4 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<float4*>(dst + 16 * m) =
            make_float4(acc[m][q][0], acc[m][q][1], acc[m][q][2], acc[m][q][3]);
    }
  }
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
