// Backward of SLA for gfx950 with the block mask held fixed.
//
// "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable
// Sparse-Linear Attention" (English abstract: the kernel supports both the
// forward and the backward pass).  With O = O_s + Y W^T the gradients are
// (per head, rows r of query block i, tokens t of key block j):
//   dY = dO W,  dW = sum_r dO_r^T Y_r,  D_r = dO_r . O_s,r = dO_r . O_r - dY_r . Y_r
//   sparse (critical pairs):  P = exp(S - lse), dP = dO V^T, dS = P (dP - D),
//       dV += P^T dO, dK += scale dS^T Q, dQ += scale dS K
//   linear (rows with den > 0):  dn = dY / den, dd = -(dY . Y) / den,
//       dphi(q) = H_i dn + dd Z_i, dQ += dphi(q) phi'(q),
//       dH_i = phi(Q_i)^T dN_i, dZ_i = phi(Q_i)^T dd_i,
//       dh_j, dz_j = sums of dH_i, dZ_i over the rows i for which j is marginal,
//       dphi(k_t) = dh_j v_t + dz_j, dK += dphi(k) phi'(k), dV += phi(K_j) dh_j
// Deterministic: every reduction has a fixed order, no atomics.
//
// Kernels here: the query-side preparation (dY, D, dN, dd and the dW
// partials), the KV-major sparse + linear dK / dV kernel, the Q-major sparse +
// linear dQ kernel, the fixed-order dW reduction and the W transpose.
#include "sla_device.h"
#include "sla_internal.h"

namespace sla {

// ---------------------------------------------------------------------------
// w_transpose: wT[c][o] = W[o][c]
// ---------------------------------------------------------------------------
__global__ void w_transpose_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wT,
                                   int D) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= D * D) return;
  const int c = e / D, o = e % D;
  wT[e] = w[static_cast<size_t>(o) * D + c];
}

// ---------------------------------------------------------------------------
// bwd_prep: one workgroup (4 waves) per run of consecutive query blocks
// (blocks b0 .. b1 - 1 of the flattened (batch x head, block) order; there are
// `parts` runs of nearly equal length).  Per query block i:
//   dY^T[c][r] = sum_o W[o][c] dO[r][o]             (wave: rows half qh, c half ch)
//   D_r = dO_r . O_r - dY_r . Y_r,  dd_r = -(dY_r . Y_r) / den_r
//   dN[r][c] = dY[r][c] / den_r     (bf16, staged in LDS and stored whole rows
//                                    per instruction)
//   dW^T partial += Y_i^T dO_i     (one 32 x 32 tile set per wave, fp32)
// and at the end the run's dW^T partial is written for the fixed-order
// reduction.  Rows r >= valid_len and rows with den = 0 get dN = 0 and
// dd = 0, so every linear gradient built from them (dQ in bwd_q, dH / dZ in
// the state builder) is zero; padded rows read as zero and add nothing to dW.
// W^T is copied into LDS once per workgroup; per block the dO and Y tiles
// arrive by asynchronous copies (whole rows per instruction, through buffer
// resources that end at valid_len) and O in 16 contiguous bytes per lane.
// Both products of a block read their operands from these tiles: the dY^T
// product takes the dO rows, the dW product takes Y^T and dO^T by transpose
// reads.  (Rows loaded one per lane had made the texture-address unit the
// limit: one address pass per row touched.)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_prep_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ wT, const float* __restrict__ den,
    const uint16_t* __restrict__ y, float* __restrict__ dsum, float* __restrict__ ddel,
    uint16_t* __restrict__ dn, float* __restrict__ dwp, long long nblocks, int parts, int N,
    int L, int T, bool linear, float gate) {
  constexpr int HP = D + 8;    // dN row pitch
  constexpr int NCC = D / 16;
  constexpr int NT = D / 64;   // 32-wide tiles per wave in each half
  constexpr int TPW = (D / 32) * (D / 32) / 4;   // dW^T tiles per wave
  constexpr int OC = kBlock * D / 8 / 256;       // 16-byte O pieces per thread
  __shared__ __attribute__((aligned(16))) uint16_t hs[D * D];     // W^T[c][o], swizzled
  // the dO tile (swizzled, unpadded) for the products, then dN[r][c] (pitch HP)
  __shared__ __attribute__((aligned(16))) uint16_t dns[64 * HP];
  __shared__ __attribute__((aligned(16))) uint16_t ys[64 * D];    // Y tile, swizzled
  __shared__ float red_oo[64];                                    // dO . O per row
  __shared__ float red_yy[2][64];                                 // dY . Y per c half and row

  const int w = static_cast<int>(xcd_remap(blockIdx.x, gridDim.x));
  const long long b0 = nblocks * w / parts, b1 = nblocks * (w + 1) / parts;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, hl = lane >> 5;
  const int qh = wave & 1, ch = wave >> 1;
  const int rloc = 32 * qh + n32;
  const uint32_t rbytes = static_cast<uint32_t>(L) * D * 2;
  {
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wT, D * D * 2);
#pragma unroll
    for (int r0 = 0; r0 < D; r0 += 64) copy_swz_buf<D, 4>(wrs, r0, hs + r0 * D, wave, lane);
  }
  f32x16 dwa[TPW];
#pragma unroll
  for (int x = 0; x < TPW; ++x) dwa[x] = f32x16{};

  for (long long b = b0; b < b1; ++b) {
    const int i = static_cast<int>(b % T);
    const long long bh = b / T;
    const size_t head = static_cast<size_t>(bh) * N * D;
    const int row = i * kBlock + rloc;   // < N always; rows >= valid_len read as zero
    const bool valid = row < L;
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dO + head, rbytes);
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(o + head, rbytes);
    const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + head, rbytes);
    copy_swz_buf<D, 4>(drs, i * kBlock, dns, wave, lane);   // dO tile, swizzled (unpadded)
    copy_swz_buf<D, 4>(yrs, i * kBlock, ys, wave, lane);    // Y tile, swizzled
    // O in 16 contiguous bytes per lane (row e / (D / 8), chunk e % (D / 8)),
    // for dO . O by rows
    u32x4 oc[OC];
#pragma unroll
    for (int u = 0; u < OC; ++u) {
      const int e = tid + 256 * u;
      oc[u] = buf_ld16(ors, static_cast<uint32_t>((i * kBlock + e / (D / 8)) * D + 8 * (e % (D / 8))) * 2u, 0);
    }
    const float dn_r = (linear && valid) ? den[bh * N + row] : 0.f;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed
    __syncthreads();

    // dY^T tiles for c in [D/2 ch, D/2 ch + D/2): A = W^T rows, B = dO rows
    // (k = o = 16 cc + 8 hl + s), both from LDS
    f32x16 dyt[NT];
    {
      bf16x8 dof[NCC];
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) dof[cc] = as_bf16x8(ld16(dns + swz_off<D>(rloc, 16 * cc + 8 * hl)));
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        dyt[ct] = f32x16{};
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc)
          dyt[ct] = mfma32(as_bf16x8(ld16(hs + swz_off<D>((D / 2) * ch + 32 * ct + n32, 16 * cc + 8 * hl))),
                           dof[cc], dyt[ct]);
#pragma unroll
        for (int e = 0; e < 16; ++e) dyt[ct][e] *= gate;   // dY of the ungated Y (gate 1: exact)
      }
    }
    // dW^T[c][o] += sum_r Y[r][c] dO[r][o]: A = Y^T, B = dO^T, both by transpose reads (k = r)
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
      const int tt = wave * TPW + x;
      const int ct = tt / (D / 32), ot = tt % (D / 32);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        dwa[x] = mfma32(swz_op32_tr<D>(ys, 16 * kk, 32 * ct, lane), swz_op32_tr<D>(dns, 16 * kk, 32 * ot, lane),
                        dwa[x]);
    }
    // dO . O by rows: each lane's chunks, summed over the D / 8 lanes of a row
#pragma unroll
    for (int u = 0; u < OC; ++u) {
      const int e = tid + 256 * u;
      const int r = e / (D / 8), c8 = e % (D / 8);
      const u32x4 dz4 = ld16(dns + swz_off<D>(r, 8 * c8));
      float pr = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
        pr = __fmaf_rn(bf16_to_f32(static_cast<uint16_t>(u4_elem(dz4, s2))),
                       bf16_to_f32(static_cast<uint16_t>(u4_elem(oc[u], s2))), pr);
#pragma unroll
      for (int m = 1; m < D / 8; m <<= 1) pr += __shfl_xor(pr, m);
      if (c8 == 0) red_oo[r] = pr;
    }
    // dY . Y partial row dots over this lane's c values (the lane's Y pieces,
    // columns 8 e4 + 4 hl .. + 3 of each tile, from the Y tile)
    float p_yy = 0.f;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const u32x2 yv = ld8(ys + swz_off<D>(rloc, (D / 2) * ch + 32 * ct + 8 * e4 + 4 * hl));
#pragma unroll
        for (int x = 0; x < 4; ++x) p_yy = __fmaf_rn(dyt[ct][4 * e4 + x], bf16_to_f32(u4_half(yv, x)), p_yy);
      }
    p_yy += __shfl_xor(p_yy, 32);
    if (hl == 0) red_yy[ch][rloc] = p_yy;
    __syncthreads();   // the dO and Y tiles read by every wave
    const float s_oo = red_oo[rloc];
    const float s_yy = red_yy[0][rloc] + red_yy[1][rloc];
    const bool lin = valid && dn_r > 0.f;
    const float rden = lin ? 1.0f / dn_r : 0.f;
    const float dd_r = lin ? -s_yy * rden : 0.f;
    if (ch == 0 && hl == 0) {
      dsum[bh * N + row] = valid ? s_oo - s_yy : 0.f;
      ddel[bh * N + row] = dd_r;
    }
    // dN = dY / den (bf16) into LDS, then to global memory from there
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int c0 = (D / 2) * ch + 32 * ct + 8 * e4 + 4 * hl;
        const u32x2 v = {pack_bf16x2(dyt[ct][4 * e4] * rden, dyt[ct][4 * e4 + 1] * rden),
                         pack_bf16x2(dyt[ct][4 * e4 + 2] * rden, dyt[ct][4 * e4 + 3] * rden)};
        st8(&dns[rloc * HP + c0], v);
      }
    __syncthreads();
    {
      // the block's dN rows, 16 contiguous bytes per lane (whole rows per
      // instruction instead of one row per lane)
      uint16_t* dblk = dn + head + static_cast<size_t>(i) * kBlock * D;
#pragma unroll
      for (int u = 0; u < kBlock * D / 8 / 256; ++u) {
        const int e = tid + 256 * u;
        const int r = e / (D / 8), c8 = e % (D / 8);
        st16(dblk + static_cast<size_t>(r) * D + 8 * c8, ld16(&dns[r * HP + 8 * c8]));
      }
    }
    __syncthreads();   // dns read by every wave before the next block's copies
  }
  // the run's dW^T partial, transposed storage dW^T[c][o] (lanes on consecutive o)
  float* out = dwp + static_cast<size_t>(w) * D * D;
#pragma unroll
  for (int x = 0; x < TPW; ++x) {
    const int tt = wave * TPW + x;
    const int ct = tt / (D / 32), ot = tt % (D / 32);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 32 * ct + 8 * (e / 4) + 4 * hl + (e % 4);
      out[static_cast<size_t>(c) * D + 32 * ot + n32] = dwa[x][e];
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_q: one workgroup per query block i; dQ = the sparse part over the
// critical key blocks plus the linear part:
//   S^T = K Q^T, P^T = exp2(S^T scale log2e - lse log2e), dP^T = V dO^T,
//   dS^T = P^T (dP^T - D), dQ_s = scale dS K
//   dphi(q)^T[a][r] = sum_c H_i[a][c] dN[r][c] + dd_r Z_i[a],
//   dQ_l[r][a] = dphi(q)[r][a] phi'(q[r][a])
// Waves (kh, qh) as in the forward; dS^T's result tile is the A operand of
// dS K directly (k index permuted) and K_j is read a second time from the
// same LDS tile with transpose reads.  K_j and V_j are double-buffered with
// the next block's loads in flight during the current block's MFMAs.  H_i^T
// and Z_i are copied into the buffers the last key block leaves free; the
// linear part is computed in the layout of the query rows (lane = row, so
// phi'(q) comes from the Q fragments already in registers) and transposed
// through LDS onto the sparse part.
// ---------------------------------------------------------------------------
template <int D>
struct BqCfg {
  static constexpr int kTile = 64 * D;                 // one K or V tile (bf16), swizzled
  static constexpr int NCC = D / 16, NAT = D / 32;
};

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ dsum,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ lut_cnt,
    const uint16_t* __restrict__ dn, const float* __restrict__ ddel,
    const uint16_t* __restrict__ hst, const float* __restrict__ zst, bool linear, bool hglobal,
    float* __restrict__ dq, int N, int L, int T, float scale) {
  using C = BqCfg<D>;
  // separate arrays, named statically by every access: the compiler can tell
  // the LDS reads from the copies in flight
  __shared__ __attribute__((aligned(16))) uint16_t kb0[C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t kb1[C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t vb1[C::kTile];
  __shared__ __attribute__((aligned(16))) float zq[2 * D];   // Z_i (two parts)

  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int i = wg % T;
  const long long bh = wg / T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave & 1, qh = wave >> 1;
  const int n32 = lane & 31, hl = lane >> 5;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int row = i * kBlock + 32 * qh + n32;
  const bool valid = row < L;
  const float sl2 = scale * kLog2e;

  bf16x8 qf[C::NCC], dof[C::NCC];
  {
    const uint16_t* qr = q + head + static_cast<size_t>(row) * D + 8 * hl;
    const uint16_t* dr = dO + head + static_cast<size_t>(row) * D + 8 * hl;
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc) {
      qf[cc] = valid ? as_bf16x8(ld16(qr + 16 * cc)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      dof[cc] = valid ? as_bf16x8(ld16(dr + 16 * cc)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
  // padded rows: zero Q and dO and an infinite lse make P = 0 and dS = 0
  const float lse2 = valid ? lse[bh * N + row] * kLog2e : INFINITY;
  const float dsv = valid ? dsum[bh * N + row] : 0.f;
  const int cnt = lut_cnt[bh * T + i];
  const int32_t* lrow = lut + (bh * T + i) * static_cast<long long>(T);
  // the list in a register (entry 64 g + l in lane l), read with readlane
  int lutv = lane < cnt ? lrow[lane] : 0;
  auto block_at = [&](int n) { return __builtin_amdgcn_readlane(lutv, n & 63); };
  // ascending lists: only the last block can be the padded one
  const int jl = cnt == 0 ? 0 : lrow[cnt - 1];
  const bool mlast = (jl + 1) * kBlock > L;

  f32x16 acc[C::NAT];
#pragma unroll
  for (int at = 0; at < C::NAT; ++at) acc[at] = f32x16{};

  // K_j, V_j by asynchronous buffer->LDS copies into swizzled tiles; the
  // resources end at valid_len, so rows of the padded block past it are zero
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + head, static_cast<uint32_t>(L) * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + head, static_cast<uint32_t>(L) * D * 2);
  auto copy_kv = [&](int n, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
    const int jb = block_at(n);
    copy_swz_buf<D, 4>(krs, jb * kBlock, kd, wave, lane);
    copy_swz_buf<D, 4>(vrs, jb * kBlock, vd, wave, lane);
  };
  // H_i^T (bf16 D x D, swizzled 64-row tiles) and Z_i for the linear part go
  // into the buffers the last key block leaves free: rows 0..63 of H_i^T into
  // its K buffer, rows 64..127 (D = 128) into its V buffer.
  const size_t hslot = static_cast<size_t>(bh) * T + (hglobal ? 0 : i);
  auto copy_h = [&](uint16_t* h0, uint16_t* h1) __attribute__((always_inline)) {
    if (!linear) return;
    const __amdgpu_buffer_rsrc_t hrs = make_rsrc(hst + hslot * D * D, D * D * 2);
    copy_swz_buf<D, 4>(hrs, 0, h0, wave, lane);
    if constexpr (D > 64) copy_swz_buf<D, 4>(hrs, 64, h1, wave, lane);
    if (wave == 0 && lane < D / 2) {
      const __amdgpu_buffer_rsrc_t zrs = make_rsrc(zst + hslot * 2 * D, 2 * D * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(zrs, (__attribute__((address_space(3))) void*)(zq),
                                               16, 16 * lane, 0, 0, 0);
    }
  };

  // Byte offsets into a swizzled tile.  Row read of key 32 kh + n32 at
  // head-dim index 16 cc + 8 hl: rowb0 ^ (cc << 5).  Permuted transpose read
  // at key rows 32 kh + 16 h (+ 8 for the upper half), columns 32 at:
  // (trb0 ^ (at << 6)) + 32 D h, upper half ^ (16 D + 16).  (The XOR swizzle
  // touches only the chunk bits, which these identities use.)
  const uint32_t rowb0 = 2u * swz_off<D>(32 * kh + n32, 8 * hl);
  const uint32_t trb0 = 2u * swz_off<D>(32 * kh + 4 * hl + ((lane & 15) >> 2),
                                        16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  auto row16 = [&](const uint16_t* t, uint32_t boff) __attribute__((always_inline)) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + boff));
  };
  auto tr16 = [&](const uint16_t* t, uint32_t boff) __attribute__((always_inline)) {
    const char* p = reinterpret_cast<const char*>(t);
    return as_bf16x8(lds_tr4(reinterpret_cast<const uint16_t*>(p + boff)),
                     lds_tr4(reinterpret_cast<const uint16_t*>(p + (boff ^ (16u * D + 16u)))));
  };
  // one key block from (kt, vt); the next one is copied into (kn, vn), or
  // H_i^T and Z_i after the last one
  auto step = [&](int n, const uint16_t* kt, const uint16_t* vt, uint16_t* kn, uint16_t* vn,
                  bool masked) __attribute__((always_inline)) {
    if (((n + 1) & 63) == 0 && n + 1 < cnt) {
      const int e = n + 1 + lane;   // the next 64 entries of the list
      lutv = e < cnt ? lrow[e] : 0;
    }
    if (n + 1 < cnt)
      copy_kv(n + 1, kn, vn);
    else
      copy_h(kn, vn);
    // the offsets pass through an empty asm each step, so the per-read XORs
    // are formed next to their reads instead of occupying registers
    uint32_t rb = rowb0, tb = trb0;
    asm("" : "+v"(rb), "+v"(tb));
    f32x16 st = {}, dpt = {};
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc) {
      st = mfma32(row16(kt, rb ^ (cc << 5)), qf[cc], st);
      dpt = mfma32(row16(vt, rb ^ (cc << 5)), dof[cc], dpt);
    }
    // B operands of dS K (K[keys][a] by transpose reads, keys in the permuted
    // order of the S^T tile), read before the exponentials so their latency
    // overlaps them
    bf16x8 bo[C::NAT][2];
#pragma unroll
    for (int at = 0; at < C::NAT; ++at)
#pragma unroll
      for (int h = 0; h < 2; ++h) bo[at][h] = tr16(kt, (tb ^ (at << 6)) + 32u * D * h);
    float dsf[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) dsf[e] = __builtin_amdgcn_exp2f(__fmaf_rn(st[e], sl2, -lse2));
    if (masked) {   // keys of the padded last block past valid_len
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = jl * kBlock + 32 * kh + 8 * (e / 4) + 4 * hl + (e % 4);
        if (key >= L) dsf[e] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) dsf[e] *= dpt[e] - dsv;
    const bf16x8 ds[2] = {cvt_bf16x8(dsf), cvt_bf16x8(dsf + 8)};
    // dQ[q][a] += dS[q][keys] K[keys][a]
#pragma unroll
    for (int at = 0; at < C::NAT; ++at)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[at] = mfma32(ds[h], bo[at][h], acc[at]);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed
    __syncthreads();
  };

  if (cnt == 0) {
    copy_h(kb0, vb0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    copy_kv(0, kb0, vb0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int n = 0; n < cnt; n += 2) {
      step(n, kb0, vb0, kb1, vb1, mlast && n + 1 == cnt);
      if (n + 1 < cnt) step(n + 1, kb1, vb1, kb0, vb0, mlast && n + 2 == cnt);
    }
  }
  // merge the key halves: wave (kh, qh) finishes the tiles at = NH kh .. NH kh + NH - 1
  // and hands the others to its partner (other kh); then add the linear part.
  // The last block's buffers hold the exchange (waves 0, 1 in its K buffer,
  // 2, 3 in its V buffer), the other ones H_i^T, then the linear part.
  constexpr int NH = C::NAT / 2;
  const bool odd = cnt & 1;   // the last block (cnt - 1) was read from kb0 / vb0
                              // (cnt = 0: H_i^T is in kb0 / vb0 as well)
  float* exq = reinterpret_cast<float*>(qh ? (odd ? vb0 : vb1) : (odd ? kb0 : kb1));
  const uint16_t* ht0 = odd ? kb1 : kb0;   // H_i^T rows 0..63
  const uint16_t* ht1 = odd ? vb1 : vb0;   // H_i^T rows 64..127
  float* lq = reinterpret_cast<float*>(qh ? (odd ? vb1 : vb0) : (odd ? kb1 : kb0));
  float* exo = exq + kh * NH * 16 * 64;
  const float* exp_ = exq + (kh ^ 1) * NH * 16 * 64;
  // the linear part's operands: this lane's dN row (B operand, k = c) and dd
  bf16x8 dnf[C::NCC];
  float ddr = 0.f;
  if (linear) {
    const uint16_t* dr = dn + head + static_cast<size_t>(row) * D + 8 * hl;
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc)
      dnf[cc] = valid ? as_bf16x8(ld16(dr + 16 * cc)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    ddr = valid ? ddel[bh * N + row] : 0.f;
  }
  __syncthreads();
  f32x16 fin[NH];
  if (kh == 0) {
#pragma unroll
    for (int x = 0; x < NH; ++x) {
      fin[x] = acc[x];
#pragma unroll
      for (int e = 0; e < 16; ++e) exo[(x * 16 + e) * 64 + lane] = acc[NH + x][e];
    }
  } else {
#pragma unroll
    for (int x = 0; x < NH; ++x) {
      fin[x] = acc[NH + x];
#pragma unroll
      for (int e = 0; e < 16; ++e) exo[(x * 16 + e) * 64 + lane] = acc[x][e];
    }
  }
  // linear part of this wave's tiles, transposed: lane = row 32 qh + n32,
  // element e = column a = 32 (NH kh + x) + 8 (e/4) + 4 hl + e%4
  f32x16 lin[NH];
  if (linear) {
#pragma unroll
    for (int x = 0; x < NH; ++x) {
      const int at = NH * kh + x;
      lin[x] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < C::NCC; ++cc) {
        const uint16_t* ht = 16 * cc < 64 ? ht0 : ht1;
        lin[x] = mfma32(swz_op32_tr<D>(ht, (16 * cc) % 64, 32 * at, lane), dnf[cc], lin[x]);
      }
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        // phi'(q) for columns 32 at + 16 p2 + 8 (e4 % 2) + 4 hl .. + 3 (e4 = 2 p2, 2 p2 + 1)
        // (kh is uniform but not a constant: both candidates are read with
        // static indices and passed through an empty asm before the select,
        // otherwise the compiler turns the select into an indexed access and
        // moves the Q fragments to scratch memory)
        u32x4 q0 = __builtin_bit_cast(u32x4, qf[2 * x + p2]);
        u32x4 q1 = __builtin_bit_cast(u32x4, qf[2 * (NH + x) + p2]);
        asm("" : "+v"(q0), "+v"(q1));
        u32x2 qe, qo;
        row_halves(kh ? q1 : q0, qe, qo);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e4 = 2 * p2 + h;
          const int a0 = 32 * at + 8 * e4 + 4 * hl;
#pragma unroll
          for (int x4 = 0; x4 < 4; ++x4) {
            const float z = zq[a0 + x4] + zq[D + a0 + x4];
            const float g = lin[x][4 * e4 + x4] + ddr * z;
            lin[x][4 * e4 + x4] = g * phi_prime(bf16_to_f32(u4_half(h ? qo : qe, x4)));
          }
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();   // the exchange is visible, every wave is done with H_i^T
  // The linear part goes to rows of fp32 in the freed H_i^T buffer of this
  // query half (row r at lq + r D, columns XOR-swizzled by row in 16-byte
  // steps so that the 32 rows of a store fall on different banks); each wave
  // reads back only what it wrote, so no barrier is needed before the reads.
  auto lq_at = [&](int r, int a) { return r * D + (a ^ ((r & (D / 4 - 1)) << 2)); };
  if (linear) {
#pragma unroll
    for (int x = 0; x < NH; ++x)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int a0 = 32 * (NH * kh + x) + 8 * e4 + 4 * hl;
        *reinterpret_cast<f32x4*>(lq + lq_at(n32, a0)) =
            f32x4{lin[x][4 * e4], lin[x][4 * e4 + 1], lin[x][4 * e4 + 2], lin[x][4 * e4 + 3]};
      }
  }
  // lane holds dQ[q = 32 qh + 8 (e/4) + 4 hl + e%4][a = 32 at + n32]
#pragma unroll
  for (int x = 0; x < NH; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int qlh = 8 * (e / 4) + 4 * hl + (e % 4);   // row within the half
      const int a = 32 * (NH * kh + x) + n32;
      const float sparse = scale * (fin[x][e] + exp_[(x * 16 + e) * 64 + lane]);
      const float lpart = linear ? lq[lq_at(qlh, a)] : 0.f;
      const int qr = i * kBlock + 32 * qh + qlh;
      dq[head + static_cast<size_t>(qr) * D + a] = qr < L ? lpart + sparse : 0.f;
    }
}

// ---------------------------------------------------------------------------
// bwd_kv: one workgroup per key block j; loops over the query blocks for which
// j is critical (column list), then adds the linear-branch gradients.
// Eight waves in two roles that share the staged Q_i / dO_i tiles: waves 0-3
// accumulate dV (S -> P -> P^T dO), waves 4-7 accumulate dK (S, dP -> dS ->
// dS^T Q).  Within a role, wave (kh, qh) owns keys 32 kh .. 32 kh + 31 of the
// block and queries 32 qh .. 32 qh + 31 of each query block.  S = Q K^T and
// dP = dO V^T take K_j, V_j from registers and Q_i, dO_i rows from LDS; the
// products over queries take P or dS straight from the S / dP result tiles
// (k index permuted) and read dO_i or Q_i from the same LDS tiles with
// transpose reads, so only the natural tiles are staged.
// Q_i, dO_i and the rows' lse / D values arrive through asynchronous
// buffer->LDS copies (Q_i, dO_i into XOR-swizzled tiles), double-buffered in
// separate arrays so that the next query block's copies overlap the current
// one's products.  The resources end at valid_len: the padded rows of the
// last query block arrive as zeros (Q = dO = 0 and D = 0 there, so they add
// nothing to dV and, with dP = 0, nothing to dK).
// Everything else the block needs -- K_j, V_j, dh_j^T and dz_j -- is copied
// into LDS asynchronously when the workgroup starts; the loop waits only for
// K_j, V_j and the first query block (each wave keeps one of K_j or V_j in
// registers as its B operands), while dh_j^T and dz_j, needed only by the
// linear epilogue, land during the first step.  Within a step each wave reads
// all of its operands for the S / dP product and the transpose-read operands
// of the product over queries before the P hand-off, so their latency
// overlaps the exponentials and the barrier.  After the loop the two query
// halves are merged so that every wave finishes two of the four 32-column
// tiles.
// ---------------------------------------------------------------------------
template <int D>
struct BkvCfg {
  static constexpr int kTile = 64 * D;                  // one Q or dO tile (bf16), swizzled
  static constexpr int NCC = D / 16, NCT = D / 32;
};

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_kv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ dsum,
    const int32_t* __restrict__ col, const int32_t* __restrict__ col_cnt,
    const uint16_t* __restrict__ dh, const float* __restrict__ dz, bool linear, bool hglobal,
    float* __restrict__ dk, float* __restrict__ dv, int N, int L, int T, float scale) {
  using C = BkvCfg<D>;
  // the streamed buffers are separate arrays, named statically by every
  // access, so the compiler can tell the LDS reads from the copies in flight
  // (Q_i tile, then the dO_i tile, in one array per stage)
  __shared__ __attribute__((aligned(16))) uint16_t qd0[2 * C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t qd1[2 * C::kTile];
  __shared__ __attribute__((aligned(16))) float lb0[128];   // lse [64] then D [64] of the rows
  __shared__ __attribute__((aligned(16))) float lb1[128];
  __shared__ __attribute__((aligned(16))) uint16_t ksw[64 * D];   // K_j, swizzled
  __shared__ __attribute__((aligned(16))) uint16_t vsw[64 * D];   // V_j
  __shared__ __attribute__((aligned(16))) uint16_t dhs[D * D];    // dh_j^T, swizzled
  __shared__ __attribute__((aligned(16))) float dzs[2 * D];       // dz_j
  __shared__ __attribute__((aligned(16))) float psh[4 * 16 * 64];  // P per (kh, qh)

  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int j = wg % T;
  const long long bh = wg / T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool role_dk = wave >= 4;               // uniform per wave
  const int kh = wave & 1, qh = (wave >> 1) & 1;
  const int n32 = lane & 31, hl = lane >> 5;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int kloc = 32 * kh + n32;               // this lane's key within the block
  const int key = j * kBlock + kloc;
  const bool kv_ok = key < L;                   // padded keys: zero operands (their P is masked too)
  const float sl2 = scale * kLog2e;

  // asynchronous copies of K_j, V_j (rows past valid_len are never used
  // unmasked), dh_j^T and dz_j
  const int cnt = col_cnt[bh * T + j];
  const int32_t* crow = col + (bh * T + j) * static_cast<long long>(T);
  // the list in a register (entry 64 g + l in lane l), read with readlane
  int colv = lane < cnt ? crow[lane] : 0;
  auto block_at = [&](int n) { return __builtin_amdgcn_readlane(colv, n & 63); };

  // K_j and V_j into LDS (keys past valid_len arrive as zero)
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + head, static_cast<uint32_t>(L) * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + head, static_cast<uint32_t>(L) * D * 2);
  copy_swz_buf<D, 8>(krs, j * kBlock, ksw, wave, lane);
  copy_swz_buf<D, 8>(vrs, j * kBlock, vsw, wave, lane);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + head, static_cast<uint32_t>(L) * D * 2);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dO + head, static_cast<uint32_t>(L) * D * 2);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lse + bh * N, static_cast<uint32_t>(L) * 4);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(dsum + bh * N, static_cast<uint32_t>(L) * 4);
  // Q_i, dO_i tiles into qd (8 waves share the copies) and the rows' lse / D values
  auto copy_q = [&](int n, uint16_t* qd, float* ld) __attribute__((always_inline)) {
    const int ib = block_at(n);
    copy_swz_buf<D, 8>(qrs, ib * kBlock, qd, wave, lane);
    copy_swz_buf<D, 8>(drs, ib * kBlock, qd + C::kTile, wave, lane);
    // lane l writes base + 16 l: lse to ld[0..63] (wave 0), D to ld[64..127] (wave 1)
    const uint32_t off = static_cast<uint32_t>(ib * kBlock + 4 * lane) * 4u;
    if (wave == 0 && lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)(ld),
                                               16, off, 0, 0, 0);
    if (wave == 1 && lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (__attribute__((address_space(3))) void*)(ld + 64),
                                               16, off, 0, 0, 0);
  };

  f32x16 acc[C::NCT];   // dV (role 0) or the unscaled dK (role 1)
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct) acc[ct] = f32x16{};

  if (cnt > 0) copy_q(0, qd0, lb0);
  // dz_j and dh_j^T (for the linear epilogue) are issued last and not waited
  // for here: the first step's end waits for them
  constexpr int kDhCopies = D * D / 4096;   // dh^T copy instructions per wave
  if (linear) {
    const size_t hslot = static_cast<size_t>(bh) * T + (hglobal ? 0 : j);
    if (wave == 7 && lane < D / 2) {
      const __amdgpu_buffer_rsrc_t zrs = make_rsrc(dz + hslot * 2 * D, 2 * D * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(zrs, (__attribute__((address_space(3))) void*)(dzs),
                                               16, 16 * lane, 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t hrs = make_rsrc(dh + hslot * D * D, D * D * 2);
#pragma unroll
    for (int r0 = 0; r0 < D; r0 += 64) copy_swz_buf<D, 8>(hrs, r0, dhs + r0 * D, wave, lane);
    __builtin_amdgcn_s_waitcnt(0xF70 | kDhCopies);   // all but the dh^T copies have landed
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  // a barrier that does not wait for the dh^T copies
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // B operands of S (dV role: K_j rows) or dP (dK role: V_j rows), k =
  // head-dim index 16 cc + 8 hl + s.  Read in one asm block that waits for
  // its own reads (outputs early-clobbered: a read's result must not land in
  // a later read's address register): the compiler would otherwise make these
  // reads wait for every copy in flight, the dh^T copies included.
  bf16x8 bf[C::NCC];
  {
    const uint16_t* fsrc = role_dk ? vsw : ksw;
    uint32_t fa[C::NCC];
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc)
      fa[cc] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(fsrc + swz_off<D>(kloc, 16 * cc + 8 * hl)));
    u32x4 fz[C::NCC];
    if constexpr (C::NCC == 8) {
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\t"
          "ds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
          "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)"
          : "=&v"(fz[0]), "=&v"(fz[1]), "=&v"(fz[2]), "=&v"(fz[3]), "=&v"(fz[4]), "=&v"(fz[5]),
            "=&v"(fz[6]), "=&v"(fz[7])
          : "v"(fa[0]), "v"(fa[1]), "v"(fa[2]), "v"(fa[3]), "v"(fa[4]), "v"(fa[5]), "v"(fa[6]),
            "v"(fa[7])
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
          : "=&v"(fz[0]), "=&v"(fz[1]), "=&v"(fz[2]), "=&v"(fz[3])
          : "v"(fa[0]), "v"(fa[1]), "v"(fa[2]), "v"(fa[3])
          : "memory");
    }
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc)
      bf[cc] = kv_ok ? as_bf16x8(fz[cc]) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }


  const bool tail_key = key >= L;
  const bool tail_blk = (j + 1) * kBlock > L;   // uniform: the padded last key block
  // one query block from (qt: Q_i then dO_i, lt); the next one is copied into (qn, ln)
  auto step = [&](int n, const uint16_t* qt, const float* lt, uint16_t* qn,
                  float* ln) __attribute__((always_inline)) {
    if (((n + 1) & 63) == 0 && n + 1 < cnt) {
      const int e = n + 1 + lane;   // the next 64 entries of the list
      colv = e < cnt ? crow[e] : 0;
    }
    if (n + 1 < cnt) copy_q(n + 1, qn, ln);
    // dV role: S = Q K^T and P, handed to the dK wave of the same (kh, qh)
    // through LDS; dK role meanwhile: dP = dO V^T.  Both result tiles have
    // lane = key, element e = query 32 qh + 8 (e/4) + 4 hl + e%4.
    const uint16_t* asrc = qt + (role_dk ? C::kTile : 0);   // Q_i or dO_i rows
    bf16x8 av[C::NCC];
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc)
      av[cc] = as_bf16x8(ld16(asrc + swz_off<D>(32 * qh + n32, 16 * cc + 8 * hl)));
    f32x16 sd = {};
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc) sd = mfma32(av[cc], bf[cc], sd);
    // B operands of the products over queries (dO_i for dV, Q_i for dK) by
    // transpose reads, query index in the permuted order of the S tile;
    // read before the hand-off so their latency overlaps it
    const uint16_t* bsrc = qt + (role_dk ? 0 : C::kTile);
    bf16x8 bo[C::NCT][2];
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int h = 0; h < 2; ++h) bo[ct][h] = swz_op32_tr_perm<D>(bsrc, 32 * qh + 16 * h, 32 * ct, lane);
    float pf[16];
    float* pw = psh + (wave & 3) * 16 * 64;   // [e / 4][lane][e % 4] of this (kh, qh)
    if (!role_dk) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lt[32 * qh + 8 * e4 + 4 * hl]);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          pf[4 * e4 + x] = __builtin_amdgcn_exp2f(__fmaf_rn(sd[4 * e4 + x], sl2, -l4[x] * kLog2e));
      }
      if (tail_blk) {   // keys past valid_len: no probability mass
#pragma unroll
        for (int e = 0; e < 16; ++e) pf[e] = tail_key ? 0.f : pf[e];
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<f32x4*>(&pw[(e4 * 64 + lane) * 4]) =
            f32x4{pf[4 * e4], pf[4 * e4 + 1], pf[4 * e4 + 2], pf[4 * e4 + 3]};
    }
    // P visible to the dK waves: LDS writes done, then a barrier that does
    // not wait for the next block's copies (the asm also keeps the compiler
    // from moving LDS accesses across it)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (role_dk) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&lt[64 + 32 * qh + 8 * e4 + 4 * hl]);
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&pw[(e4 * 64 + lane) * 4]);
#pragma unroll
        for (int x = 0; x < 4; ++x) pf[4 * e4 + x] = p4[x] * (sd[4 * e4 + x] - d4[x]);
      }
    }
    const bf16x8 xb[2] = {cvt_bf16x8(pf), cvt_bf16x8(pf + 8)};
    // dV[key][c] += P^T dO  or  dK[key][a] += dS^T Q
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[ct] = mfma32(xb[h], bo[ct][h], acc[ct]);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed
    __syncthreads();
  };
  for (int n = 0; n < cnt; n += 2) {
    step(n, qd0, lb0, qd1, lb1);
    if (n + 1 < cnt) step(n + 1, qd1, lb1, qd0, lb0);
  }

  // ---- merge the query halves: wave (role, qh, kh) finishes the tiles
  // ct = 2 qh, 2 qh + 1 and hands the other two to its partner (other qh).
  // lane holds X[key = 32 kh + 8 (e/4) + 4 hl + e%4][c = 32 ct + n32]
  constexpr int NH = C::NCT / 2;
  // exchange area [wave][NH][16][64] floats: two waves per streamed tile
  auto exw = [&](int w) {
    uint16_t* b = ((w >> 2) ? qd1 : qd0) + ((w >> 1) & 1) * C::kTile;
    return reinterpret_cast<float*>(b) + (w & 1) * NH * 16 * 64;
  };
  float* exo = exw(wave);
  const float* exq = exw(wave ^ 2);
  // (qh is uniform per wave; both branches index acc statically)
  f32x16 fin[NH];
  if (qh == 0) {
#pragma unroll
    for (int x = 0; x < NH; ++x) {
      fin[x] = acc[x];
#pragma unroll
      for (int e = 0; e < 16; ++e) exo[(x * 16 + e) * 64 + lane] = acc[NH + x][e];
    }
  } else {
#pragma unroll
    for (int x = 0; x < NH; ++x) {
      fin[x] = acc[NH + x];
#pragma unroll
      for (int e = 0; e < 16; ++e) exo[(x * 16 + e) * 64 + lane] = acc[x][e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NH; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float sum = fin[x][e] + exq[(x * 16 + e) * 64 + lane];
      fin[x][e] = role_dk ? scale * sum : sum;
    }
  if (linear) {
    // A operand rows t = key: phi(K_j)[t][a] (dV role) or V_j[t][c] (dK role), from registers
    bf16x8 af[C::NCC];
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc) {
      if (role_dk) {
        af[cc] = bf[cc];
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          af[cc][s2] = static_cast<__bf16>(kv_ok ? phi(static_cast<float>(bf[cc][s2])) : 0.f);
      }
    }
#pragma unroll
    for (int x = 0; x < NH; ++x) {
      const int ct = NH * qh + x;
      f32x16 lin = {};
#pragma unroll
      for (int cc = 0; cc < C::NCC; ++cc) {
        // dV role: dV_lin[t][c] = sum_a phi(K)[t][a] dh[a][c], B = dh^T[c][a .. a + 7] (row)
        // dK role: dphi(K)[t][a] = sum_c V[t][c] dh[a][c],     B = dh^T[c .. c + 7][a] (transpose read)
        const bf16x8 b = role_dk ? swz_op32_tr<D>(dhs, 16 * cc, 32 * ct, lane)
                                 : as_bf16x8(ld16(dhs + swz_off<D>(32 * ct + n32, 16 * cc + 8 * hl)));
        lin = mfma32(af[cc], b, lin);
      }
      // lane holds X[t = 32 kh + 8 (e/4) + 4 hl + e%4][n = 32 ct + n32]
      const int a = 32 * ct + n32;
      if (role_dk) {
        const float dza = dzs[a] + dzs[D + a];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const u32x2 k4 = swz_col4<D>(ksw, 32 * kh + 8 * e4, 32 * ct, lane);   // K[t .. t + 3][a]
#pragma unroll
          for (int x4 = 0; x4 < 4; ++x4)
            fin[x][4 * e4 + x4] += (lin[4 * e4 + x4] + dza) * phi_prime(bf16_to_f32(u4_half(k4, x4)));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) fin[x][e] += lin[e];
      }
    }
  }
  float* out = role_dk ? dk : dv;
#pragma unroll
  for (int x = 0; x < NH; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tt = j * kBlock + 32 * kh + 8 * (e / 4) + 4 * hl + (e % 4);
      out[head + static_cast<size_t>(tt) * D + 32 * (NH * qh + x) + n32] = tt < L ? fin[x][e] : 0.f;
    }
}

// ---------------------------------------------------------------------------
// dW: fixed-order reduction of the partials that bwd_prep writes (stored transposed, entry e = c D + o):
// workgroup of 256 threads per 64 entries; thread group g (of 4) sums
// partials g, g + 4, ... in order, and the four group sums are added in order;
// times the linear-output gate (1 for SLA); written to dW[o][c].
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float* __restrict__ part,
                                                        float* __restrict__ dw, int DD, int D,
                                                        int parts, float gate) {
  __shared__ float red[4][64];
  const int tid = threadIdx.x, g = tid >> 6;
  const int e = blockIdx.x * 64 + (tid & 63);
  float s = 0.f;
  if (e < DD) {
    int p = g;
    for (; p + 28 < parts; p += 32) {   // eight loads in flight, summed in order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[static_cast<size_t>(p + 4 * u) * DD + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; p < parts; p += 4) s += part[static_cast<size_t>(p) * DD + e];
  }
  red[g][tid & 63] = s;
  __syncthreads();
  if (g == 0 && e < DD)
    dw[(e % D) * D + e / D] = gate * (((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_w_transpose(const Dims& d, const uint16_t* w, uint16_t* wT, hipStream_t s) {
  hipLaunchKernelGGL(w_transpose_kernel, dim3((d.D * d.D + 255) / 256), dim3(256), 0, s, w, wT, d.D);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const Dims& d, const uint16_t* o, const uint16_t* dO,
                           const uint16_t* wT, const float* den, const uint16_t* y, bool linear,
                           float* dsum, float* ddel, uint16_t* dn, float* dw_part, hipStream_t s) {
  const long long nblocks = d.BH() * d.T;
  const int parts = dw_parts(d);
  if (d.D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(parts), dim3(256), 0, s, o, dO, wT, den, y, dsum,
                       ddel, dn, dw_part, nblocks, parts, d.N, d.L, d.T, linear, d.gate);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(parts), dim3(256), 0, s, o, dO, wT, den, y, dsum,
                       ddel, dn, dw_part, nblocks, parts, d.N, d.L, d.T, linear, d.gate);
  return hipGetLastError();
}

hipError_t launch_bwd_q(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dO, const float* lse, const float* dsum,
                        const int32_t* lut, const int32_t* lut_cnt, const uint16_t* dn,
                        const float* ddel, const uint16_t* hst, const float* zst, bool linear,
                        float* dq, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(d.BH() * d.T));
  if (d.D == 128)
    hipLaunchKernelGGL(bwd_q_kernel<128>, grid, dim3(256), 0, s, q, k, v, dO, lse, dsum, lut,
                       lut_cnt, dn, ddel, hst, zst, linear, d.global, dq, d.N, d.L, d.T, d.scale);
  else
    hipLaunchKernelGGL(bwd_q_kernel<64>, grid, dim3(256), 0, s, q, k, v, dO, lse, dsum, lut,
                       lut_cnt, dn, ddel, hst, zst, linear, d.global, dq, d.N, d.L, d.T, d.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* lse, const float* dsum,
                         const int32_t* col, const int32_t* col_cnt, const uint16_t* dh,
                         const float* dz, bool linear, float* dk, float* dv, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(d.BH() * d.T));
  if (d.D == 128)
    hipLaunchKernelGGL(bwd_kv_kernel<128>, grid, dim3(512), 0, s, q, k, v, dO, lse, dsum, col,
                       col_cnt, dh, dz, linear, d.global, dk, dv, d.N, d.L, d.T, d.scale);
  else
    hipLaunchKernelGGL(bwd_kv_kernel<64>, grid, dim3(512), 0, s, q, k, v, dO, lse, dsum, col,
                       col_cnt, dh, dz, linear, d.global, dk, dv, d.N, d.L, d.T, d.scale);
  return hipGetLastError();
}

hipError_t launch_dw_reduce(const Dims& d, const float* part, float* dw, hipStream_t s) {
  const int dd = d.D * d.D;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((dd + 63) / 64), dim3(256), 0, s, part, dw, dd, d.D,
                     dw_parts(d), d.gate);
  return hipGetLastError();
}

}  // namespace sla
