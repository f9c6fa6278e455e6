// Forward preparation kernels for gfx950: per-key-block linear-attention
// states, block mean pooling, the compressed score map and the three-way
// classifier (critical / marginal / negligible per query block), plus the
// list builders that turn a block mask into the index lists the attention
// kernels consume.
//
// Method: "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable
// Sparse-Linear Attention" (English abstract; method section, steps 1-4 of the
// technical framework).  Classification ranks key blocks on a mean-pooled
// (block-compressed) score map, the selection family described in the
// abstract of "Trainable Log-linear Sparse Attention for Efficient Diffusion
// Transformers".
#include "sla_device.h"
#include "sla_internal.h"

namespace sla {

// ---------------------------------------------------------------------------
// Column sums over a 64-token block (z, the pooled means) use one fixed
// order everywhere: 16 chunks of 4 consecutive tokens, each summed in token
// order from 0, then the 16 chunk sums combined as a balanced binary tree.
// pool_kernel and kv_state_kernel share it, so the pooled K of the forward is
// bit-identical to the one the standalone pool/score entry point computes.
// ---------------------------------------------------------------------------
constexpr int kSumChunks = 16;

// p[c * stride], c = 0..15, added as a balanced binary tree
__device__ __forceinline__ float tree16(const float* p, int stride) {
  float l1[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) l1[c] = p[(2 * c) * stride] + p[(2 * c + 1) * stride];
  const float a = (l1[0] + l1[1]) + (l1[2] + l1[3]);
  const float b = (l1[4] + l1[5]) + (l1[6] + l1[7]);
  return a + b;
}

// ---------------------------------------------------------------------------
// kv_state: for key block j of head bh
//   h_j^T[c][a] = sum_t v_t[c] * phi(k_t)[a],  z_j[a] = sum_t phi(k_t)[a],
//   kbar_j[a]   = mean_t k_t[a]            (valid tokens t only)
// h^T and z are written as bf16 in the "K-tiled" layout the aggregation GEMM
// reads as its A operand: states[bh][j / 4][n][j % 4], n = c*D + a for h^T,
// n = D*D + a for bf16(z), n = D*D + D + a for bf16(z - bf16(z)).  One
// workgroup handles 8 consecutive key blocks (two planes of 4); every lane
// writes the 4 block values of one state entry of a plane as one 8-byte
// store, so a wave writes whole 512-byte runs; it has one
// wave per 32x32 tile of h^T (16 waves for D = 128), so K and V are read
// once.  The tiles are staged row-major (a plain copy, phi applied on the
// way) and both MFMA operands, which run over tokens, come from LDS
// transpose reads.  phi(k) is rounded to bf16 once and the same rounded
// values feed h and z.  The next block's rows are loaded during the current
// block's products.
// BWD = true turns the same kernel into the backward's query-side state
// builder: Y = Q, X = dN (bf16 rows), and the vector part is weighted,
// dZ_i[a] = sum_r d_r * phi(q_r)[a] with the per-row weights d_r; no pooled
// mean is written then.
// ---------------------------------------------------------------------------
template <int D>
struct KvCfg {
  static constexpr int kTiles = (D / 32) * (D / 32);   // 32x32 tiles of h^T
  static constexpr int kThreads = kTiles * 64;         // one tile per wave
  static constexpr int kCh = 64 * D / 8 / kThreads;    // 16-byte row chunks per thread and tensor
  static constexpr int kSlices = kThreads / D;         // threads per column in the column sums
  static constexpr int kPitch = D == 128 ? 152 : 72;   // LDS row pitch (bf16), conflict-free transpose reads
};

template <int D, bool BWD>
__global__ __launch_bounds__(KvCfg<D>::kThreads) void kv_state_kernel(
    const uint16_t* __restrict__ ysrc, const uint16_t* __restrict__ xsrc,
    const float* __restrict__ wrow, float* __restrict__ kbar, uint16_t* __restrict__ states,
    int N, int L, int T, int Tp) {
  using C = KvCfg<D>;
  constexpr int P = C::kPitch;
  constexpr int NB = D * D + 2 * D;
  constexpr int CPS = kSumChunks / C::kSlices;   // chunks summed per thread
  __shared__ __attribute__((aligned(16))) uint16_t pk[64 * P];   // phi(Y)[t][a], bf16
  __shared__ __attribute__((aligned(16))) uint16_t xs[64 * P];   // X[t][c]
  __shared__ __attribute__((aligned(16))) uint16_t ks[BWD ? 8 : 64 * P];   // Y[t][a] raw (pooled mean)
  __shared__ float zpart[kSumChunks][D];
  __shared__ float kpart[BWD ? 1 : kSumChunks][D];
  __shared__ uint16_t zst[2 * D * 8];
  __shared__ float wts[kBlock];

  const int groups = Tp / 8;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / groups;
  const int g = wg % groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n32 = lane & 31;
  const int hl = lane >> 5;
  const size_t head = static_cast<size_t>(bh) * N * D;

  u32x4 rk[C::kCh], rv[C::kCh];
  auto load = [&](int j) {
#pragma unroll
    for (int u = 0; u < C::kCh; ++u) {
      const int e = tid + C::kThreads * u;
      const int tok = j * kBlock + e / (D / 8);
      if (j < T && tok < L) {
        const size_t off = head + static_cast<size_t>(tok) * D + 8 * (e % (D / 8));
        rk[u] = ld16(ysrc + off);
        rv[u] = ld16(xsrc + off);
      } else {
        rk[u] = u32x4{0u, 0u, 0u, 0u};
        rv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  const int ct = wave / (D / 32), at = wave % (D / 32);   // this wave's 32x32 tile of h^T
  const int sa = tid % D, sl = tid / D;                     // column-sum unit: column, slice
  // bf16 pairs of (block 2p, block 2p+1) per result entry, four blocks at a time
  uint32_t stash[16][2];
  uint16_t* out = states + (static_cast<size_t>(bh) * groups + g) * NB * 8;   // planes 2g, 2g + 1
  load(g * 8);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int j = g * 8 + jj;
    // stage the rows (invalid tokens are zero in all three tiles)
#pragma unroll
    for (int u = 0; u < C::kCh; ++u) {
      const int e = tid + C::kThreads * u;
      const int r = e / (D / 8), c8 = e % (D / 8);
      const int row = r * P + 8 * c8;
      st16(&xs[row], rv[u]);
      if constexpr (!BWD) st16(&ks[row], rk[u]);
      const bool ok = j < T && j * kBlock + r < L;
      float f[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
        f[s2] = ok ? phi(bf16_to_f32(static_cast<uint16_t>(u4_elem(rk[u], s2)))) : 0.f;
      st16(&pk[row], __builtin_bit_cast(u32x4, cvt_bf16x8(f)));
    }
    if constexpr (BWD) {
      if (tid < kBlock) {
        const int tok = j * kBlock + tid;
        wts[tid] = (j < T && tok < L) ? wrow[static_cast<size_t>(bh) * N + tok] : 0.f;
      }
    }
    __syncthreads();
    if (jj < 7) load(j + 1);
    {
      // C[m = c][n = a] = sum_t X[t][c] phi(Y)[t][a]: both operands by transpose reads (k = t)
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma32(lds_op32_tr<false>(xs, P, 16 * kk, 32 * ct, lane),
                     lds_op32_tr<false>(pk, P, 16 * kk, 32 * at, lane), acc);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t hb = f32_to_bf16(acc[i]);
        if (jj & 1)
          stash[i][(jj >> 1) & 1] |= hb << 16;
        else
          stash[i][(jj >> 1) & 1] = hb;
      }
      if ((jj & 3) == 3) {   // blocks jj-3 .. jj: one 8-byte half of each 16-byte entry
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * ct + 8 * (i / 4) + 4 * hl + (i % 4);
          const int a = 32 * at + n32;
          st8(out + static_cast<size_t>(jj >> 2) * NB * 4 + (static_cast<size_t>(c) * D + a) * 4,
              u32x2{stash[i][0], stash[i][1]});
        }
      }
    }
    // chunk sums of z (weighted in BWD mode) and of the raw rows
#pragma unroll
    for (int cc = 0; cc < CPS; ++cc) {
      const int c = sl * CPS + cc;
      float zs = 0.f, ksum = 0.f;
#pragma unroll
      for (int t = 4 * c; t < 4 * c + 4; ++t) {
        if constexpr (BWD) {
          zs = __fmaf_rn(wts[t], bf16_to_f32(pk[t * P + sa]), zs);
        } else {
          zs += bf16_to_f32(pk[t * P + sa]);
          ksum += bf16_to_f32(ks[t * P + sa]);
        }
      }
      zpart[c][sa] = zs;
      if constexpr (!BWD) kpart[c][sa] = ksum;
    }
    __syncthreads();
    if (tid < D) {
      const int a = tid;
      const float zs = tree16(&zpart[0][a], D);
      const uint16_t zh = f32_to_bf16(zs);
      zst[a * 8 + jj] = zh;
      zst[(D + a) * 8 + jj] = f32_to_bf16(zs - bf16_to_f32(zh));
      if constexpr (!BWD) {
        if (j < T) {
          const int nvalid = min(kBlock, L - j * kBlock);
          kbar[(static_cast<size_t>(bh) * T + j) * D + a] =
              tree16(&kpart[0][a], D) / static_cast<float>(nvalid);
        }
      }
    }
  }

  __syncthreads();   // zst complete
  for (int e = tid; e < 2 * D; e += C::kThreads) {
    const u32x4 zz = ld16(&zst[e * 8]);
    st8(out + (static_cast<size_t>(D) * D + e) * 4, u32x2{zz[0], zz[1]});
    st8(out + static_cast<size_t>(NB) * 4 + (static_cast<size_t>(D) * D + e) * 4, u32x2{zz[2], zz[3]});
  }
}

// ---------------------------------------------------------------------------
// pool: xbar[bh][i][a] = mean of the valid rows of block i, in the column-sum
// order above.  One workgroup (2 D threads) per block: thread (column group of
// 8, chunk c) loads its chunk's four rows with 16-byte loads.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(2 * D) void pool_kernel(const uint16_t* __restrict__ x,
                                                     float* __restrict__ xbar, int N, int L,
                                                     int T) {
  __shared__ float part[kSumChunks][D];
  const long long r = blockIdx.x;
  const long long bh = r / T;
  const int i = static_cast<int>(r % T);
  const int tid = threadIdx.x;
  const int cg = tid % (D / 8), c = tid / (D / 8);
  // rows past valid_len read as zero through the bounded resource (no branches)
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + static_cast<size_t>(bh) * N * D,
                                              static_cast<uint32_t>(L) * D * 2);
  const int nvalid = min(kBlock, L - i * kBlock);
  u32x4 v[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    v[t] = buf_ld16(rs, static_cast<uint32_t>((i * kBlock + 4 * c + t) * D + 8 * cg) * 2u, 0);
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) s[e] += bf16_to_f32(static_cast<uint16_t>(u4_elem(v[t], e)));
    part[c][8 * cg + e] = s[e];
  }
  __syncthreads();
  if (tid < D) xbar[static_cast<size_t>(r) * D + tid] = tree16(&part[0][tid], D) / static_cast<float>(nvalid);
}

// ---------------------------------------------------------------------------
// scores[bh][i][j] = (sum_a qbar_i[a] * kbar_j[a]) * scale: fp32 fused
// multiply-adds in order a = 0..D-1, then one multiply by the scale.
// 64 x 64 tile per workgroup.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ qbar,
                                                     const float* __restrict__ kbar,
                                                     float* __restrict__ scores, int T,
                                                     float scale) {
  constexpr int A4 = D / 4;   // float4 columns of a row
  constexpr int AC = 8;       // float4 columns staged at a time (32 of the a)
  // one float4 of row padding: the 16 rows a wave reads fall on distinct banks.
  // (Staging 32 of the a at a time keeps the LDS per workgroup at 18 KB, so
  // eight workgroups share a compute unit; the order of the fused
  // multiply-adds, a = 0 .. D - 1, is the same.)
  __shared__ f32x4 qs[64][AC + 1];
  __shared__ f32x4 ks[64][AC + 1];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const f32x4* qh = reinterpret_cast<const f32x4*>(qbar + static_cast<size_t>(bh) * T * D);
  const f32x4* kh = reinterpret_cast<const f32x4*>(kbar + static_cast<size_t>(bh) * T * D);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float acc[4][4] = {};
  for (int c0 = 0; c0 < A4; c0 += AC) {
    __syncthreads();   // the previous columns are consumed
    for (int e = threadIdx.x; e < 64 * AC; e += 256) {
      const int r = e / AC, a4 = e % AC;
      qs[r][a4] = (i0 + r < T) ? qh[static_cast<size_t>(i0 + r) * A4 + c0 + a4] : zero;
      ks[r][a4] = (j0 + r < T) ? kh[static_cast<size_t>(j0 + r) * A4 + c0 + a4] : zero;
    }
    __syncthreads();
#pragma unroll 2
    for (int a4 = 0; a4 < AC; ++a4) {
      f32x4 qv[4], kv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[r] = qs[ty + 16 * r][a4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kv[c] = ks[tx + 16 * c][a4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {   // a = 4 (c0 + a4) + 0 .. 3, in order
          acc[r][c] = __fmaf_rn(qv[r][0], kv[c][0], acc[r][c]);
          acc[r][c] = __fmaf_rn(qv[r][1], kv[c][1], acc[r][c]);
          acc[r][c] = __fmaf_rn(qv[r][2], kv[c][2], acc[r][c]);
          acc[r][c] = __fmaf_rn(qv[r][3], kv[c][3], acc[r][c]);
        }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
      if (i < T && j < T) scores[(static_cast<size_t>(bh) * T + i) * T + j] = __fmul_rn(acc[r][c], scale);
    }
}

// ---------------------------------------------------------------------------
// classify: one wave per row (bh, i).  A key block's sort key is the pair
// (code, j): code is the fp32 score mapped to an unsigned value that grows as
// the score falls (-0 folded onto +0), j the block index.  Positions
// 0..k_c-1 of the ascending order are critical, T-k_n..T-1 negligible, the
// rest marginal.  Instead of sorting the row, the key at each of the two
// boundary positions is found by a radix select on the code (four 8-bit
// digits, a 256-bin histogram per wave in LDS), and keys whose code equals
// the boundary code are ranked by index with ballots.  Writes the mask row;
// optionally the ascending critical list and the marginal bit row.  Rows i
// in [T, Tp) only clear their bit row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t descending_code(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);   // -0 -> +0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// Radix select over the keys one wave holds: key 64 u + lane has code
// code[u] and takes part where ok[u].  Finds the key at position r (0-based)
// of the ascending (code, index) order: its code, and its rank among the
// keys with that code (those are ordered by index).  Four passes over 8-bit
// digits, each a 256-bin histogram in the wave's own LDS words (one wave's
// LDS accesses execute in order, so no barrier is needed), a prefix sum over
// the bins and a ballot for the bin that holds position r.
template <int NC>
__device__ __forceinline__ void wave_select(const uint32_t (&code)[NC], const bool (&ok)[NC], int r,
                                            uint32_t* hist, int lane, uint32_t& code_at,
                                            int& tie_at) {
  uint32_t prefix = 0u, pmask = 0u;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 24 - 8 * pass;
    *reinterpret_cast<u32x4*>(&hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < NC; ++u)
      if (ok[u] && (code[u] & pmask) == prefix) atomicAdd(&hist[(code[u] >> sh) & 255u], 1u);
    const u32x4 hv = *reinterpret_cast<const u32x4*>(&hist[4 * lane]);
    const int sum = static_cast<int>(hv[0] + hv[1] + hv[2] + hv[3]);
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    // the first lane whose bins reach past position r holds the digit
    const int src = __builtin_ctzll(__ballot(incl > r));
    int below = incl - sum, digit = 4 * lane;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (below + static_cast<int>(hv[k]) > r) break;
      below += static_cast<int>(hv[k]);
      ++digit;
    }
    digit = __shfl(digit, src);
    below = __shfl(below, src);
    r -= below;
    prefix |= static_cast<uint32_t>(digit) << sh;
    pmask |= 0xFFu << sh;
  }
  code_at = prefix;
  tie_at = r;
}

// One wave writes row i of the mask, and optionally its ascending critical
// list with the count and its marginal bit row (word-major), from per-chunk
// flags: key block 64 u + lane is critical where crit[u], negligible where
// negl[u] (and not critical), marginal otherwise; ok[u]: the block exists.
template <int NC>
__device__ __forceinline__ void wave_emit(const bool (&ok)[NC], const bool (&crit)[NC],
                                          const bool (&negl)[NC], int8_t* __restrict__ mask,
                                          int32_t* __restrict__ lut, int32_t* __restrict__ lut_cnt,
                                          uint32_t* __restrict__ rbits, long long bh, int i, int T,
                                          int Tp, int nch, int lane) {
  const int words = Tp / 32;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int8_t* mrow = mask + (bh * T + i) * T;
  int32_t* lrow = lut ? lut + (bh * T + i) * T : nullptr;
  uint32_t* brow = rbits ? rbits + bh * words * Tp + i : nullptr;   // word w at brow[w * Tp]
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    if (u < nch) {
      const int j = 64 * u + lane;
      if (ok[u]) mrow[j] = crit[u] ? 1 : (negl[u] ? -1 : 0);
      const unsigned long long bcrit = __ballot(crit[u]);
      if (lrow && crit[u]) lrow[cnt + __popcll(bcrit & lt)] = j;
      cnt += __popcll(bcrit);
      if (brow) {
        const unsigned long long bm = __ballot(ok[u] && !crit[u] && !negl[u]);
        if (lane == 0) {
          brow[(2 * u) * Tp] = static_cast<uint32_t>(bm);
          if (2 * u + 1 < words) brow[(2 * u + 1) * Tp] = static_cast<uint32_t>(bm >> 32);
        }
      }
    }
  }
  if (lut_cnt && lane == 0) lut_cnt[bh * T + i] = cnt;
}

// NCH: 64-wide chunks a lane walks (at least ceil(T / 64))
template <int NCH>
__global__ __launch_bounds__(256) void classify_kernel(const float* __restrict__ scores,
                                                       int8_t* __restrict__ mask,
                                                       int32_t* __restrict__ lut,
                                                       int32_t* __restrict__ lut_cnt,
                                                       uint32_t* __restrict__ rbits, int T,
                                                       int Tp, int rows, int kc, int kn) {
  __shared__ __attribute__((aligned(16))) uint32_t hists[4][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * 4 + wave;
  const long long bh = blockIdx.y;
  const int words = Tp / 32;
  if (i >= rows) return;
  if (i >= T) {
    if (rbits)
      for (int w = lane; w < words; w += 64) rbits[(bh * words + w) * Tp + i] = 0u;
    return;
  }
  uint32_t* hist = hists[wave];
  const int nch = (T + 63) / 64;
  const float* row = scores + (bh * T + i) * T;
  uint32_t code[NCH];
  bool ok[NCH];
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int j = 64 * u + lane;
    ok[u] = u < nch && j < T;
    code[u] = ok[u] ? descending_code(row[j]) : 0u;
  }
  // critical: positions <= k_c - 1; negligible: positions >= T - k_n
  uint32_t cc = 0u, cn = 0xFFFFFFFFu;
  int qc = -1, qn = 1 << 30;
  if (kc > 0) wave_select(code, ok, kc - 1, hist, lane, cc, qc);
  if (kn > 0) wave_select(code, ok, T - kn, hist, lane, cn, qn);
  const unsigned long long lt = (1ull << lane) - 1ull;
  bool crit[NCH], negl[NCH];
  int tc = 0, tn = 0;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const bool eqc = ok[u] && kc > 0 && code[u] == cc;
    const bool eqn = ok[u] && kn > 0 && code[u] == cn;
    const unsigned long long bc = __ballot(eqc), bn = __ballot(eqn);
    const int tie_c = tc + __popcll(bc & lt), tie_n = tn + __popcll(bn & lt);
    tc += __popcll(bc);
    tn += __popcll(bn);
    crit[u] = ok[u] && kc > 0 && (code[u] < cc || (eqc && tie_c <= qc));
    negl[u] = ok[u] && kn > 0 && (code[u] > cn || (eqn && tie_n >= qn));
  }
  wave_emit(ok, crit, negl, mask, lut, lut_cnt, rbits, bh, i, T, Tp, nch, lane);
}



// ---------------------------------------------------------------------------
// Two-level selection, after the abstract of "Trainable Log-linear Sparse
// Attention for Efficient Diffusion Transformers": key blocks are grouped G
// at a time, a group's coarse key is the mean of its valid rows, the first
// `keep` groups by coarse score (descending, index ascending) are kept and the
// last n_g negligible; only the blocks of the kept groups get fine scores, and
// the first k_c of them (fine score descending, index ascending) are critical.
// ---------------------------------------------------------------------------
// kgbar[g] = sum over the blocks j of group g of n_j kbar[j] / sum n_j, with
// n_j the valid rows of block j (blocks ascending, fp32).
__global__ __launch_bounds__(256) void group_means_kernel(const float* __restrict__ kbar,
                                                          float* __restrict__ kgbar, int T, int D,
                                                          int G, int Tg, int L) {
  const long long bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;   // (group, column)
  if (e >= Tg * D) return;
  const int g = e / D, a = e % D;
  const int j1 = min((g + 1) * G, T);
  float acc = 0.f;
  int n = 0;
  for (int j = g * G; j < j1; ++j) {
    const int nj = min(kBlock, L - j * kBlock);   // >= 1: only the last block is short
    acc = __fmaf_rn(static_cast<float>(nj), kbar[(bh * T + j) * D + a], acc);
    n += nj;
  }
  kgbar[(bh * Tg + g) * D + a] = __fdiv_rn(acc, static_cast<float>(n));
}

// s * (q . k) over D entries, accumulated in index order with fused
// multiply-adds (the order of the compressed score map)
__device__ __forceinline__ float ordered_score(const float* q, const float* __restrict__ k, int D,
                                               float scale) {
  float acc = 0.f;
  for (int a = 0; a < D; a += 4) {
    const f32x4 qv = *reinterpret_cast<const f32x4*>(q + a);
    const f32x4 kv = *reinterpret_cast<const f32x4*>(k + a);
    acc = __fmaf_rn(qv[0], kv[0], acc);
    acc = __fmaf_rn(qv[1], kv[1], acc);
    acc = __fmaf_rn(qv[2], kv[2], acc);
    acc = __fmaf_rn(qv[3], kv[3], acc);
  }
  return __fmul_rn(acc, scale);
}

// coarse map alone: one workgroup per (row i, bh)
__global__ __launch_bounds__(256) void coarse_scores_kernel(const float* __restrict__ qbar,
                                                            const float* __restrict__ kgbar,
                                                            float* __restrict__ coarse, int T,
                                                            int D, int Tg, float scale) {
  __shared__ __attribute__((aligned(16))) float qs[128];
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  for (int a = threadIdx.x; a < D; a += 256) qs[a] = qbar[(bh * T + i) * D + a];
  __syncthreads();
  for (int g = threadIdx.x; g < Tg; g += 256)
    coarse[(bh * T + i) * Tg + g] = ordered_score(qs, kgbar + (bh * Tg + g) * D, D, scale);
}

// One wave per row (bh, i).  Level 1: the coarse keys of the Tg groups
// (computed, or read from coarse_in); the keys at positions keep - 1 and
// Tg - n_g of their ascending (code, index) order are found by the radix
// select, which marks the kept groups (positions < keep) and the negligible
// ones (positions >= Tg - n_g).  Level 2: the blocks of the kept groups,
// compacted in block order into candidate slots, get fine keys (computed, or
// read from scores_in); the key at position k_c - 1 of their order bounds
// the critical blocks.  Blocks of negligible groups that are not critical are
// negligible, the rest marginal; the row is written like the flat
// classifier's.  NC: 64-wide chunks a lane walks (at least ceil(T / 64)).
template <int NC>
__global__ __launch_bounds__(256) void classify_hier_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kgbar,
    const float* __restrict__ kbar, const float* __restrict__ coarse_in,
    const float* __restrict__ scores_in, int8_t* __restrict__ mask, int32_t* __restrict__ lut,
    int32_t* __restrict__ lut_cnt, uint32_t* __restrict__ rbits, int T, int Tp, int D, int G,
    int Tg, int keep, int ng, int kc, float scale, int rows) {
  __shared__ __attribute__((aligned(16))) uint32_t hists[4][256];
  __shared__ __attribute__((aligned(16))) float qsh[4][128];
  __shared__ uint8_t gfl[4][kMaxT];    // per group: bit 0 kept, bit 1 negligible
  __shared__ int16_t candj[4][kMaxT];  // candidate slot -> block
  __shared__ int8_t crs[4][kMaxT];     // per block: critical
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * 4 + wave;
  const long long bh = blockIdx.y;
  if (i >= rows) return;
  if (i >= T) {
    const int words = Tp / 32;
    if (rbits)
      for (int w = lane; w < words; w += 64) rbits[(bh * words + w) * Tp + i] = 0u;
    return;
  }
  uint32_t* hist = hists[wave];
  float* qs = qsh[wave];
  const bool given = coarse_in != nullptr;
  if (!given)
    for (int a = lane; a < D; a += 64) qs[a] = qbar[(bh * T + i) * D + a];
  __builtin_amdgcn_wave_barrier();
  const unsigned long long lt = (1ull << lane) - 1ull;

  // ---- level 1: groups
  const int ngc = (Tg + 63) / 64;
  uint32_t gcode[NC];
  bool gok[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int g = 64 * u + lane;
    gok[u] = u < ngc && g < Tg;
    gcode[u] = gok[u] ? descending_code(given ? coarse_in[(bh * T + i) * Tg + g]
                                              : ordered_score(qs, kgbar + (bh * Tg + g) * D, D, scale))
                      : 0u;
  }
  uint32_t ck = 0u, cn = 0xFFFFFFFFu;
  int qk = -1, qn = 1 << 30;
  wave_select(gcode, gok, keep - 1, hist, lane, ck, qk);
  if (ng > 0) wave_select(gcode, gok, Tg - ng, hist, lane, cn, qn);
  {
    int tk = 0, tn = 0;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const bool eqk = gok[u] && gcode[u] == ck;
      const bool eqn = gok[u] && ng > 0 && gcode[u] == cn;
      const unsigned long long bk = __ballot(eqk), bn = __ballot(eqn);
      const int tie_k = tk + __popcll(bk & lt), tie_n = tn + __popcll(bn & lt);
      tk += __popcll(bk);
      tn += __popcll(bn);
      const bool kept = gok[u] && (gcode[u] < ck || (eqk && tie_k <= qk));
      const bool negl = gok[u] && ng > 0 && (gcode[u] > cn || (eqn && tie_n >= qn));
      if (gok[u]) gfl[wave][64 * u + lane] = static_cast<uint8_t>((kept ? 1 : 0) | (negl ? 2 : 0));
    }
  }
  __builtin_amdgcn_wave_barrier();

  // ---- level 2: the blocks of the kept groups into candidate slots, in
  // block order (so slot order breaks ties like block order)
  const int nch = (T + 63) / 64;
  int ncand = 0;
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    if (u < nch) {
      const int j = 64 * u + lane;
      const bool c = j < T && (gfl[wave][j / G] & 1);
      crs[wave][j] = 0;
      const unsigned long long bc = __ballot(c);
      if (c) candj[wave][ncand + __popcll(bc & lt)] = static_cast<int16_t>(j);
      ncand += __popcll(bc);
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int ncc = (ncand + 63) / 64;
  uint32_t fcode[NC];
  bool fok[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int sl = 64 * u + lane;
    fok[u] = u < ncc && sl < ncand;
    fcode[u] = 0u;
    if (fok[u]) {
      const int j = candj[wave][sl];
      fcode[u] = descending_code(given ? scores_in[(bh * T + i) * T + j]
                                       : ordered_score(qs, kbar + (bh * T + j) * D, D, scale));
    }
  }
  if (kc > 0) {
    uint32_t cc;
    int qc;
    wave_select(fcode, fok, kc - 1, hist, lane, cc, qc);
    int tc = 0;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const bool eqc = fok[u] && fcode[u] == cc;
      const unsigned long long bc = __ballot(eqc);
      const int tie_c = tc + __popcll(bc & lt);
      tc += __popcll(bc);
      if (fok[u] && (fcode[u] < cc || (eqc && tie_c <= qc))) crs[wave][candj[wave][64 * u + lane]] = 1;
    }
  }
  __builtin_amdgcn_wave_barrier();
  bool ok[NC], crit[NC], negl[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int j = 64 * u + lane;
    ok[u] = u < nch && j < T;
    crit[u] = ok[u] && crs[wave][j] != 0;
    negl[u] = ok[u] && !crit[u] && (gfl[wave][j / G] & 2);
  }
  wave_emit(ok, crit, negl, mask, lut, lut_cnt, rbits, bh, i, T, Tp, nch, lane);
}

// ---------------------------------------------------------------------------
// mask_lists: from a three-valued mask build, per row, the ascending list of
// critical key blocks and the marginal bit row; per column, the ascending
// list of query blocks for which the key block is critical and the marginal
// bit column.  Values other than +1 and 0 count as negligible.
// blockIdx.z = 0: rows, 1: columns.  Index Tp-T tail rows/columns clear bits.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mask_lists_kernel(const int8_t* __restrict__ mask,
                                                        int32_t* __restrict__ lut,
                                                        int32_t* __restrict__ lut_cnt,
                                                        uint32_t* __restrict__ rbits,
                                                        int32_t* __restrict__ col,
                                                        int32_t* __restrict__ col_cnt,
                                                        uint32_t* __restrict__ cbits, int T,
                                                        int Tp) {
  const int x = blockIdx.x;
  const long long bh = blockIdx.y;
  const bool by_col = blockIdx.z == 1;
  const int lane = threadIdx.x;
  const int words = Tp / 32;
  int32_t* list = by_col ? col : lut;
  int32_t* cnts = by_col ? col_cnt : lut_cnt;
  uint32_t* bits = by_col ? cbits : rbits;
  if (list == nullptr) return;
  uint32_t* brow = bits ? bits + bh * words * Tp + x : nullptr;   // word w at brow[w * Tp]
  if (x >= T) {
    if (brow)
      for (int w = lane; w < words; w += 64) brow[w * Tp] = 0u;
    return;
  }
  const int8_t* m = mask + bh * T * T;
  int cnt = 0;
  int32_t* lrow = list + (bh * T + x) * T;
  for (int base = 0; base < Tp; base += 64) {
    const int y = base + lane;
    int8_t val = -1;
    if (y < T) val = by_col ? m[static_cast<long long>(y) * T + x] : m[static_cast<long long>(x) * T + y];
    const bool crit = y < T && val == 1;
    const bool marg = y < T && val == 0;
    const unsigned long long bc = __ballot(crit);
    if (crit) lrow[cnt + __popcll(bc & ((1ull << lane) - 1ull))] = y;
    cnt += __popcll(bc);
    const unsigned long long bm = __ballot(marg);
    if (brow && lane == 0) {
      brow[(base / 32) * Tp] = static_cast<uint32_t>(bm);
      if (base / 32 + 1 < words) brow[(base / 32 + 1) * Tp] = static_cast<uint32_t>(bm >> 32);
    }
  }
  if (lane == 0) cnts[bh * T + x] = cnt;
}

// The column pass when T is a multiple of 4: one wave per four adjacent
// columns, each row's four mask bytes read with one aligned 32-bit load (the
// byte-per-row column reads touch 64 cache lines per instruction; this reads
// each line once for four columns).  Same lists, counts and bits as the
// column half of mask_lists_kernel.
__global__ __launch_bounds__(64) void mask_cols4_kernel(const int8_t* __restrict__ mask,
                                                        int32_t* __restrict__ col,
                                                        int32_t* __restrict__ col_cnt,
                                                        uint32_t* __restrict__ cbits, int T,
                                                        int Tp) {
  const int x0 = 4 * blockIdx.x;
  const long long bh = blockIdx.y;
  const int lane = threadIdx.x;
  const int words = Tp / 32;
  const int8_t* m = mask + bh * T * T;
  // columns x0 .. x0 + 3 < Tp; those at or past T only get cleared bits
  const int ncols = x0 + 4 <= T ? 4 : (x0 < T ? T - x0 : 0);
  int cnt[4] = {0, 0, 0, 0};
  for (int base = 0; base < Tp; base += 64) {
    const int y = base + lane;
    // x0 + 3 < T whenever ncols > 0 (T is a multiple of 4), so the word is
    // inside row y; rows past T read as all-negligible
    const uint32_t v4 = (y < T && ncols > 0)
                            ? *reinterpret_cast<const uint32_t*>(m + static_cast<long long>(y) * T + x0)
                            : 0xFFFFFFFFu;
#pragma unroll
    for (int xi = 0; xi < 4; ++xi) {
      const int x = x0 + xi;
      const int8_t val = static_cast<int8_t>((v4 >> (8 * xi)) & 0xffu);
      const bool crit = xi < ncols && val == 1;
      const bool marg = xi < ncols && val == 0;
      const unsigned long long bc = __ballot(crit);
      if (crit) col[(bh * T + x) * T + cnt[xi] + __popcll(bc & ((1ull << lane) - 1ull))] = y;
      cnt[xi] += __popcll(bc);
      const unsigned long long bm = __ballot(marg);
      if (cbits && lane == 0 && x < Tp) {
        uint32_t* brow = cbits + bh * words * Tp + x;   // word w at brow[w * Tp]
        brow[(base / 32) * Tp] = static_cast<uint32_t>(bm);
        if (base / 32 + 1 < words) brow[(base / 32 + 1) * Tp] = static_cast<uint32_t>(bm >> 32);
      }
    }
  }
  if (lane < ncols) {
    int c = cnt[0];
    c = lane == 1 ? cnt[1] : c;
    c = lane == 2 ? cnt[2] : c;
    c = lane == 3 ? cnt[3] : c;
    col_cnt[bh * T + x0 + lane] = c;
  }
}

__global__ void fill_mask_kernel(int8_t* __restrict__ mask, long long n, int8_t value) {
  for (long long e = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
       e += static_cast<long long>(gridDim.x) * blockDim.x)
    mask[e] = value;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_kv_state(const Dims& d, const uint16_t* k, const uint16_t* v, float* kbar,
                           uint16_t* states, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(d.BH() * (d.Tp / 8)));
  if (d.D == 128)
    hipLaunchKernelGGL((kv_state_kernel<128, false>), grid, dim3(KvCfg<128>::kThreads), 0, s, k, v,
                       nullptr, kbar, states, d.N, d.L, d.T, d.Tp);
  else
    hipLaunchKernelGGL((kv_state_kernel<64, false>), grid, dim3(KvCfg<64>::kThreads), 0, s, k, v,
                       nullptr, kbar, states, d.N, d.L, d.T, d.Tp);
  return hipGetLastError();
}

hipError_t launch_dstate(const Dims& d, const uint16_t* q, const uint16_t* dn, const float* ddel,
                         uint16_t* states, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(d.BH() * (d.Tp / 8)));
  if (d.D == 128)
    hipLaunchKernelGGL((kv_state_kernel<128, true>), grid, dim3(KvCfg<128>::kThreads), 0, s, q, dn,
                       ddel, nullptr, states, d.N, d.L, d.T, d.Tp);
  else
    hipLaunchKernelGGL((kv_state_kernel<64, true>), grid, dim3(KvCfg<64>::kThreads), 0, s, q, dn,
                       ddel, nullptr, states, d.N, d.L, d.T, d.Tp);
  return hipGetLastError();
}

hipError_t launch_pool(const Dims& d, const uint16_t* x, float* xbar, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(d.BH() * d.T));
  if (d.D == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, s, x, xbar, d.N, d.L, d.T);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(128), 0, s, x, xbar, d.N, d.L, d.T);
  return hipGetLastError();
}

hipError_t launch_scores(const Dims& d, const float* qbar, const float* kbar, float* scores,
                         hipStream_t s) {
  const int tiles = (d.T + 63) / 64;
  const dim3 grid(tiles, tiles, static_cast<unsigned>(d.BH()));
  if (d.D == 128)
    hipLaunchKernelGGL(scores_kernel<128>, grid, dim3(256), 0, s, qbar, kbar, scores, d.T, d.scale);
  else
    hipLaunchKernelGGL(scores_kernel<64>, grid, dim3(256), 0, s, qbar, kbar, scores, d.T, d.scale);
  return hipGetLastError();
}

hipError_t launch_classify(const Dims& d, const float* scores, int8_t* mask, int32_t* lut,
                           int32_t* lut_cnt, uint32_t* rbits, hipStream_t s) {
  const int rows = rbits ? d.Tp : d.T;
  const dim3 grid((rows + 3) / 4, static_cast<unsigned>(d.BH()));
  if (d.T <= 512)
    hipLaunchKernelGGL(classify_kernel<8>, grid, dim3(256), 0, s, scores, mask, lut, lut_cnt, rbits,
                       d.T, d.Tp, rows, d.kc, d.kn);
  else
    hipLaunchKernelGGL(classify_kernel<kMaxT / 64>, grid, dim3(256), 0, s, scores, mask, lut, lut_cnt,
                       rbits, d.T, d.Tp, rows, d.kc, d.kn);
  return hipGetLastError();
}

hipError_t launch_group_means(const Dims& d, const float* kbar, float* kgbar, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((d.Tg * d.D + 255) / 256), static_cast<unsigned>(d.BH()));
  hipLaunchKernelGGL(group_means_kernel, grid, dim3(256), 0, s, kbar, kgbar, d.T, d.D, d.G, d.Tg,
                     d.L);
  return hipGetLastError();
}

hipError_t launch_coarse_scores(const Dims& d, const float* qbar, const float* kgbar,
                                float* coarse, hipStream_t s) {
  hipLaunchKernelGGL(coarse_scores_kernel, dim3(d.T, static_cast<unsigned>(d.BH())), dim3(256), 0,
                     s, qbar, kgbar, coarse, d.T, d.D, d.Tg, d.scale);
  return hipGetLastError();
}

hipError_t launch_classify_hier(const Dims& d, const float* qbar, const float* kgbar,
                                const float* kbar, const float* coarse_in, const float* scores_in,
                                int8_t* mask, int32_t* lut, int32_t* lut_cnt, uint32_t* rbits,
                                hipStream_t s) {
  const int rows = rbits ? d.Tp : d.T;
  const dim3 grid((rows + 3) / 4, static_cast<unsigned>(d.BH()));
  if (d.T <= 512)
    hipLaunchKernelGGL(classify_hier_kernel<8>, grid, dim3(256), 0, s, qbar, kgbar, kbar, coarse_in,
                       scores_in, mask, lut, lut_cnt, rbits, d.T, d.Tp, d.D, d.G, d.Tg, d.keep,
                       d.ng, d.kc, d.scale, rows);
  else if (d.T <= 1024)
    hipLaunchKernelGGL(classify_hier_kernel<16>, grid, dim3(256), 0, s, qbar, kgbar, kbar, coarse_in,
                       scores_in, mask, lut, lut_cnt, rbits, d.T, d.Tp, d.D, d.G, d.Tg, d.keep,
                       d.ng, d.kc, d.scale, rows);
  else
    hipLaunchKernelGGL(classify_hier_kernel<kMaxT / 64>, grid, dim3(256), 0, s, qbar, kgbar, kbar,
                       coarse_in, scores_in, mask, lut, lut_cnt, rbits, d.T, d.Tp, d.D, d.G, d.Tg,
                       d.keep, d.ng, d.kc, d.scale, rows);
  return hipGetLastError();
}

hipError_t launch_mask_lists(const Dims& d, const int8_t* mask, int32_t* lut, int32_t* lut_cnt,
                             uint32_t* rbits, int32_t* col, int32_t* col_cnt, uint32_t* cbits,
                             hipStream_t s) {
  // rows (and, unless T is a multiple of 4, columns) by mask_lists_kernel
  const bool cols4 = col != nullptr && d.T % 4 == 0;
  const unsigned z = (col && !cols4) ? 2u : 1u;
  hipLaunchKernelGGL(mask_lists_kernel, dim3(d.Tp, static_cast<unsigned>(d.BH()), z), dim3(64), 0,
                     s, mask, lut, lut_cnt, rbits, col, col_cnt, cbits, d.T, d.Tp);
  if (cols4) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mask_cols4_kernel, dim3(d.Tp / 4, static_cast<unsigned>(d.BH())), dim3(64),
                       0, s, mask, col, col_cnt, cbits, d.T, d.Tp);
  }
  return hipGetLastError();
}

hipError_t launch_fill_mask(const Dims& d, int8_t* mask, int8_t value, hipStream_t s) {
  const long long n = d.BH() * d.T * d.T;
  const long long blocks = std::min<long long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_mask_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, mask,
                     n, value);
  return hipGetLastError();
}

}  // namespace sla
