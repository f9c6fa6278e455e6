// Fused SLA forward for gfx950: one workgroup per (batch, head, query block).
//
// "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable
// Sparse-Linear Attention" (English abstract; method section, steps 2-5):
// exact softmax attention over the critical key blocks, linear attention over
// the marginal ones, negligible blocks skipped, all in one kernel.  Per query
// block i of 64 rows:
//   sparse:  for every critical key block j: S = Q_i K_j^T (bf16 MFMA, fp32),
//            online softmax in base 2 with lazy rescaling, O += P V_j (P in bf16)
//   linear:  Y = (phi(Q_i) H_i) / (phi(Q_i) . Z_i)   (H_i, Z_i from the
//            aggregation kernel; bf16 MFMA, fp32)
//   fusion:  O = O_s + Y W^T
//
// Layout of the work: 4 waves, wave (kh, qh) owns key half kh (32 of the 64
// keys of every critical block) and query half qh (32 rows).  Everything is
// computed transposed (S^T = K Q^T, O^T = V^T P^T) with v_mfma_f32_32x32x16:
// then the S^T result tile, converted to bf16, is directly the B operand of
// the P V product (k index permuted identically in the V^T operand), each
// lane owns one query row, and row statistics need a single exchange between
// the two 32-lane halves.
// The loop is software-pipelined by one block: iteration n issues the S^T
// MFMAs of block n and, while they run, does the online softmax of block
// n - 1 and its P V product, so the matrix cores and the vector ALUs work at
// the same time within each wave.  K_j and V_j arrive in LDS through
// asynchronous buffer->LDS copies into XOR-swizzled row-major tiles (no
// staging registers, no LDS stores), K one iteration ahead of its use and V
// two (K tiles and V tiles have two buffers each); the V^T operand is read
// from the V tile with LDS transpose reads.  The swizzle keeps the 16-byte
// operand reads and the transpose reads spread over the LDS banks.
// The two key halves are merged at the end like split-K partial softmaxes,
// each wave finishing half of the output tiles.  H_i and Z_i for the linear
// branch are copied asynchronously into the K buffers once the last S^T tile
// has been computed.
#include "sla_device.h"
#include "sla_internal.h"

namespace sla {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* w;
  const int32_t* lut;
  const int32_t* lut_cnt;
  const uint16_t* hst;
  const float* zst;
  uint16_t* o;
  float* lse;
  float* den;
  uint16_t* y;
  int N, L, T;
  float scale_log2;
  int hglobal;   // H, Z shared by every query block (slot 0 of the head)
  float gate;    // O = O_s + gate * Y W^T
};

template <int D>
struct AttnCfg {
  static constexpr int kTile = 64 * D;             // one K or V tile (bf16 elements), swizzled
  static constexpr int kExtra = 4096;              // bytes: Z_i and the merge statistics
  static constexpr int NCT = D / 32;               // 32-row tiles of O^T per wave
  static constexpr int NCC = D / 16;               // 16-wide k chunks over the head dim
};

template <int D, bool DENSE, bool LINEAR>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs args) {
  using C = AttnCfg<D>;
  // Every buffer is its own array and every access names its array
  // statically, so the compiler can tell the LDS reads from the copies in
  // flight and does not hold the reads back until the copies land.
  __shared__ __attribute__((aligned(16))) uint16_t kb0[C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t kb1[C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t vb1[C::kTile];
  __shared__ __attribute__((aligned(16))) float extra[C::kExtra / 4];

  const int T = args.T, N = args.N, L = args.L;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int i = wg % T;
  const long long bh = wg / T;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave & 1, qh = wave >> 1;
  const int n32 = lane & 31, hl = lane >> 5;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int row = i * kBlock + 32 * qh + n32;   // this lane's query row
  const float sl2 = args.scale_log2;

  // Q fragments: B operand of S^T = K Q^T (k = head-dim index 16 cc + 8 hl + s)
  bf16x8 qf[C::NCC];
  {
    const uint16_t* qrow = args.q + head + static_cast<size_t>(row) * D + 8 * hl;
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc)
      qf[cc] = row < L ? as_bf16x8(ld16(qrow + 16 * cc)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  const int cnt = DENSE ? T : args.lut_cnt[bh * T + i];
  const int32_t* lrow = DENSE ? nullptr : args.lut + (bh * T + i) * static_cast<long long>(T);
  // the list is held in a register, entry 64 g + l in lane l for the current
  // group g = n / 64 (reloaded when the loop enters the next group): the loop
  // takes its block indices with readlane instead of a memory load
  int lutv = 0;
  if (!DENSE && lane < cnt) lutv = lrow[lane];
  auto block_at = [&](int n) { return DENSE ? n : __builtin_amdgcn_readlane(lutv, n & 63); };
  // ascending lists: only the last block can be the padded one
  const int jl = cnt == 0 ? 0 : DENSE ? cnt - 1 : lrow[cnt - 1];
  const bool mlast = (jl + 1) * kBlock > L;

  // K_j and V_j arrive through asynchronous buffer->LDS copies into swizzled
  // tiles (no staging registers).  The resources end at valid_len, so the
  // rows of the padded last block past it arrive as zeros.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(args.k + head, static_cast<uint32_t>(L) * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(args.v + head, static_cast<uint32_t>(L) * D * 2);
  auto copy_k = [&](int n, uint16_t* dst) __attribute__((always_inline)) {
    if (n < cnt) copy_swz_buf<D, 4>(krs, block_at(n) * kBlock, dst, wave, lane);
  };
  auto copy_v = [&](int n, uint16_t* dst) __attribute__((always_inline)) {
    copy_swz_buf<D, 4>(vrs, block_at(n) * kBlock, dst, wave, lane);
  };
  // in the loop, each copy instruction takes a per-lane constant offset and a
  // resource that starts at the block's first row
  uint32_t cvoff[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u) cvoff[u] = swz_copy_voff<D, 4>(wave, lane, u);
  // H_i^T (swizzled, rows 0..63 into kb0 and 64..127 into kb1) and Z_i, once
  // the K buffers are no longer read
  float* zsw = extra;   // 2 D floats
  auto copy_hz = [&]() __attribute__((always_inline)) {
    if constexpr (LINEAR) {
      const size_t hslot = static_cast<size_t>(bh) * T + (args.hglobal ? 0 : i);
      const uint16_t* hsrc = args.hst + hslot * D * D;
      copy_swz<D>(hsrc, kb0, 64, wave, 4, lane);
      if constexpr (D == 128) copy_swz<D>(hsrc + 64 * D, kb1, 64, wave, 4, lane);
      if (wave == 3 && lane < D / 2) gl_to_lds16(args.zst + hslot * 2 * D + 4 * lane, zsw);
    }
  };

  f32x16 acc[C::NCT];
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct) acc[ct] = f32x16{};
  float m_run = -INFINITY;   // running max (log2 units) of this lane's query
  float l_run = 0.f;         // partial row sum over this lane's keys

  // S^T = K Q^T for the K tile kt; K operand rows read four chunks ahead;
  // hook(cc) runs after MFMA cc (the copies of the next tiles are issued
  // there, one instruction at a time, so a wave that stalls on a full copy
  // queue does so while its MFMAs run instead of before them)
  auto s_tile = [&](const uint16_t* kt, auto&& hook) __attribute__((always_inline)) {
    constexpr int KA = C::NCC < 4 ? C::NCC : 4;
    bf16x8 ka[KA];
#pragma unroll
    for (int cc = 0; cc < KA; ++cc)
      ka[cc] = as_bf16x8(ld16(kt + swz_off<D>(32 * kh + n32, 16 * cc + 8 * hl)));
    f32x16 st = {};
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc) {
      const bf16x8 a = ka[cc % KA];
      if (cc + KA < C::NCC)
        ka[cc % KA] = as_bf16x8(ld16(kt + swz_off<D>(32 * kh + n32, 16 * (cc + KA) + 8 * hl)));
      st = mfma32(a, qf[cc], st);
      hook(cc);
    }
    return st;
  };
  auto no_hook = [](int) {};
  // online softmax of one S^T tile (base 2, lazy rescale) and O^T += V^T P^T
  // with the V tile vt; masked: the tile of the padded last key block jl
  auto soft_pv = [&](f32x16 st, const uint16_t* vt, bool masked) __attribute__((always_inline)) {
    if (masked) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = jl * kBlock + 32 * kh + 8 * (e / 4) + 4 * hl + (e % 4);
        if (key >= L) st[e] = -INFINITY;
      }
    }
    float mraw = max16(st);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw), __float_as_uint(mraw),
                                                       false, false);
      mraw = fmax_p(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // max over both lane halves
    }
    const float m_new = fmax_p(m_run, mraw * sl2);
    const bool need = m_new > m_run + 8.0f;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      if (need) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ct][e] *= alpha;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = __builtin_amdgcn_exp2f(__fmaf_rn(st[e], sl2, -mu));
      l_run += p[e];
    }
    const bf16x8 pb[2] = {cvt_bf16x8(p), cvt_bf16x8(p + 8)};
    // O^T += V^T P^T; the V^T operands come from transpose reads of the V tile
    // (keys in the permuted order of the S^T tile: k index of chunk h is keys
    // 16 h + {4 hl .. 4 hl + 3, 8 + 4 hl .. 8 + 4 hl + 3})
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[ct] = mfma32(swz_op32_tr_perm<D>(vt, 32 * kh + 16 * h, 32 * ct, lane), pb[h], acc[ct]);
  };
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed
    __syncthreads();
  };

  // Iteration n (1 <= n < cnt): K_n is in kc, V_{n-1} in vp, S^T of block
  // n - 1 in sp; K_{n+1} is copied into kn (the buffer of K_{n-1}) and V_n
  // into vn (the buffer of V_{n-2}).
  f32x16 sp;
  // (the copy instructions go between the S^T MFMAs: D / 32 for the K tile,
  // then D / 32 for the V tile, one after each of the D / 16 MFMAs)
  auto iter = [&](int n, const uint16_t* kc, uint16_t* kn, uint16_t* vn,
                  const uint16_t* vp) __attribute__((always_inline)) {
    const int jv = block_at(n);
    // entry n + 1 starts a new group of 64: the register takes the next 64
    // entries of the list (after entry n was read above)
    if (!DENSE && ((n + 1) & 63) == 0 && n + 1 < cnt) {
      const int e = n + 1 + lane;
      lutv = e < cnt ? lrow[e] : 0;
    }
    const bool kmore = n + 1 < cnt;
    const int jk = kmore ? block_at(n + 1) : 0;
    const __amdgpu_buffer_rsrc_t kr = rows_rsrc<D>(args.k + head, jk * kBlock, L);
    const __amdgpu_buffer_rsrc_t vr = rows_rsrc<D>(args.v + head, jv * kBlock, L);
    const f32x16 sn = s_tile(kc, [&](int cc) __attribute__((always_inline)) {
      if (cc < D / 32) {
        if (kmore) copy_swz_rows_one<D, 4>(kr, cvoff[cc], kn, wave, cc);
      } else {
        copy_swz_rows_one<D, 4>(vr, cvoff[cc - D / 32], vn, wave, cc - D / 32);
      }
    });
    soft_pv(sp, vp, false);
    sp = sn;
    sync();
  };

  if (cnt == 0) {
    copy_hz();
  } else {
    copy_k(0, kb0);
    sync();
    copy_k(1, kb1);
    copy_v(0, vb0);
    sp = s_tile(kb0, no_hook);
    sync();
    int n = 1;
    for (; n + 1 < cnt; n += 2) {
      iter(n, kb1, kb0, vb1, vb0);
      iter(n + 1, kb0, kb1, vb0, vb1);
    }
    if (n < cnt) iter(n, kb1, kb0, vb1, vb0);
    // last block cnt - 1: its V tile is in vb0 when cnt is odd
    copy_hz();
    if (cnt & 1)
      soft_pv(sp, vb0, mlast);
    else
      soft_pv(sp, vb1, mlast);
  }
  l_run += __shfl_xor(l_run, 32);

  // the W rows of the fusion product are loaded now, so their latency
  // overlaps the merge and the linear branch: wave (kh, qh) finishes output
  // columns o in [D/2 kh, D/2 kh + D/2), A operand W[o][16 cc + 8 hl .. + 7]
  constexpr int NCL = D / 64;   // 32-row tiles per wave in each half
  bf16x8 wf[LINEAR ? NCL : 1][C::NCC];
  if constexpr (LINEAR) {
#pragma unroll
    for (int ot = 0; ot < NCL; ++ot) {
      const uint16_t* wr = args.w + static_cast<size_t>((D / 2) * kh + 32 * ot + n32) * D + 8 * hl;
#pragma unroll
      for (int cc = 0; cc < C::NCC; ++cc) wf[ot][cc] = as_bf16x8(ld16(wr + 16 * cc));
    }
  }

  // ---- merge the two key halves (split-K style): wave (kh, qh) finishes the
  // O_s^T tiles ct = NH kh .. NH kh + NH - 1 and hands the others to its partner.
  constexpr int NH = C::NCT / 2;
  // exchange area [wave][NH][16][64] floats: waves 0, 1 in vb0, waves 2, 3 in vb1
  auto exw = [&](int w) {
    return reinterpret_cast<float*>(w >> 1 ? vb1 : vb0) + (w & 1) * NH * 16 * 64;
  };
  float* exo = exw(wave);
  const float* exp_ = exw(wave ^ 1);
  float* exm = extra + 2 * D;                                            // [wave][64]
  float* exl = exm + 4 * 64;                                             // [wave][64]
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
  exm[wave * 64 + lane] = m_run;
  exl[wave * 64 + lane] = l_run;
  __builtin_amdgcn_s_waitcnt(0);   // this wave's H / Z copies have landed
  __syncthreads();
  const bool valid_row = row < L;
  const int partner = wave ^ 1;
  {
    const float m2 = exm[partner * 64 + lane], l2 = exl[partner * 64 + lane];
    const float ms = fmaxf(m_run, m2);
    float a1 = 0.f, a2 = 0.f, inv = 0.f, lse_v = -INFINITY;
    if (ms != -INFINITY) {
      a1 = __builtin_amdgcn_exp2f(m_run - ms);
      a2 = __builtin_amdgcn_exp2f(m2 - ms);
      const float ls = a1 * l_run + a2 * l2;
      if (ls > 0.f) {
        inv = 1.0f / ls;
        lse_v = (ms + __log2f(ls)) * kLn2;
      }
    }
#pragma unroll
    for (int x = 0; x < NH; ++x)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        fin[x][e] = (a1 * fin[x][e] + a2 * exp_[(x * 16 + e) * 64 + lane]) * inv;
    if (kh == 0 && hl == 0) args.lse[bh * N + row] = valid_row ? lse_v : -INFINITY;
  }
  // lane holds O_s^T[c = 32 (NH kh + x) + 8 (e/4) + 4 hl + e%4][row]
  uint16_t* orow = args.o + head + static_cast<size_t>(row) * D;
  if constexpr (!LINEAR) {
    // O = O_s; no marginal blocks: Y = 0, den = 0
#pragma unroll
    for (int x = 0; x < NH; ++x)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int c = 32 * (NH * kh + x) + 8 * e4 + 4 * hl;
        u32x2 v = {0u, 0u};
        if (valid_row)
          v = u32x2{pack_bf16x2(fin[x][4 * e4], fin[x][4 * e4 + 1]),
                    pack_bf16x2(fin[x][4 * e4 + 2], fin[x][4 * e4 + 3])};
        st8(orow + c, v);
      }
    uint16_t* yrow = args.y + head + static_cast<size_t>(row) * D;
#pragma unroll
    for (int c = (D / 2) * kh + 8 * hl; c < (D / 2) * (kh + 1); c += 16) st16(yrow + c, u32x4{0u, 0u, 0u, 0u});
    if (kh == 0 && hl == 0) args.den[bh * N + row] = 0.f;
    return;
  } else {
    // ---- linear branch: Y^T = (H_i^T phi(Q)^T) / den, wave (kh = c half, qh) ----
    bf16x8 pq[C::NCC];
    float dpart = 0.f;
#pragma unroll
    for (int cc = 0; cc < C::NCC; ++cc) {
      const int a0 = 16 * cc + 8 * hl;   // this lane's head-dim indices a0 .. a0 + 7
      const f32x4 z0 = *reinterpret_cast<const f32x4*>(&zsw[a0]);
      const f32x4 z1 = *reinterpret_cast<const f32x4*>(&zsw[a0 + 4]);
      const f32x4 y0 = *reinterpret_cast<const f32x4*>(&zsw[D + a0]);
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(&zsw[D + a0 + 4]);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const __bf16 r = static_cast<__bf16>(phi(static_cast<float>(qf[cc][s])));
        pq[cc][s] = r;
        const float z = s < 4 ? z0[s] + y0[s] : z1[s - 4] + y1[s - 4];
        dpart += static_cast<float>(r) * z;
      }
    }
    const float den_v = dpart + __shfl_xor(dpart, 32);
    const float rden = den_v > 0.f ? 1.0f / den_v : 0.f;
    // Y^T tiles: wave (kh, qh) computes c in [D/2 kh, D/2 kh + D/2)
    // H^T row c: rows 0 .. 63 are in kb0, rows 64 .. 127 (D = 128) in kb1
    const uint16_t* hsw = (D == 128 && kh) ? kb1 : kb0;
    const int hrow0 = D == 128 ? 0 : (D / 2) * kh;
    f32x16 lin[NCL];
#pragma unroll
    for (int ct = 0; ct < NCL; ++ct) {
      lin[ct] = f32x16{};
      const int c = hrow0 + 32 * ct + n32;
#pragma unroll
      for (int cc = 0; cc < C::NCC; ++cc)
        lin[ct] = mfma32(as_bf16x8(ld16(hsw + swz_off<D>(c, 16 * cc + 8 * hl))), pq[cc], lin[ct]);
    }
    if (kh == 0 && hl == 0) args.den[bh * N + row] = valid_row ? den_v : 0.f;
    __syncthreads();   // exchange area free again: reuse it for Y (bf16 [64][D + 8])
    constexpr int YP = D + 8;
    uint16_t* ysl = reinterpret_cast<uint16_t*>(qh ? vb1 : vb0);   // rows 32 qh .. 32 qh + 31
    uint16_t* yrow = args.y + head + static_cast<size_t>(row) * D;
#pragma unroll
    for (int ct = 0; ct < NCL; ++ct)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int c = (D / 2) * kh + 32 * ct + 8 * e4 + 4 * hl;
        const uint32_t w0 = pack_bf16x2(lin[ct][4 * e4] * rden, lin[ct][4 * e4 + 1] * rden);
        const uint32_t w1 = pack_bf16x2(lin[ct][4 * e4 + 2] * rden, lin[ct][4 * e4 + 3] * rden);
        st8(ysl + n32 * YP + c, u32x2{w0, w1});
        st8(yrow + c, valid_row ? u32x2{w0, w1} : u32x2{0u, 0u});
      }
    __syncthreads();
    // ---- fusion: O^T = O_s^T + W Y^T, wave (kh = o half, qh) ----
    const uint16_t* ys = ysl + n32 * YP + 8 * hl;
#pragma unroll
    for (int ot = 0; ot < NCL; ++ot) {
      const int obase = (D / 2) * kh + 32 * ot;
      f32x16 out = {};
#pragma unroll
      for (int cc = 0; cc < C::NCC; ++cc) out = mfma32(wf[ot][cc], as_bf16x8(ld16(ys + 16 * cc)), out);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int o0 = obase + 8 * e4 + 4 * hl;
        float r[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) r[x] = out[4 * e4 + x] * args.gate + fin[ot][4 * e4 + x];
        st8(orow + o0, valid_row ? u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])}
                                 : u32x2{0u, 0u});
      }
    }
  }
}

template <int D>
static hipError_t launch_attn_t(const AttnArgs& a, unsigned grid, bool dense, bool linear,
                                hipStream_t s) {
  if (dense) {
    if (linear)
      hipLaunchKernelGGL((attn_fwd_kernel<D, true, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, true, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (linear)
      hipLaunchKernelGGL((attn_fwd_kernel<D, false, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, false, false>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const Dims& d, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* w, const int32_t* lut,
                           const int32_t* lut_cnt, bool dense, bool linear,
                           const uint16_t* hst, const float* zst, uint16_t* o, float* lse,
                           float* den, uint16_t* y, hipStream_t s) {
  AttnArgs a{q, k, v, w, lut, lut_cnt, hst, zst, o, lse, den, y, d.N, d.L, d.T,
             d.scale * kLog2e, d.global ? 1 : 0, d.gate};
  const unsigned grid = static_cast<unsigned>(d.BH() * d.T);
  if (d.D == 128) return launch_attn_t<128>(a, grid, dense, linear, s);
  return launch_attn_t<64>(a, grid, dense, linear, s);
}

}  // namespace sla
