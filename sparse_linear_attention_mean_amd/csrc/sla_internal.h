// Internal layout of the workspace / saved buffers and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sla.h"

namespace sla {

// Shapes derived from a validated sla_config.
struct Dims {
  int B, H, N, D, L;   // batch, heads, seq_len, head_dim, valid_len
  int T;               // number of 64-token blocks
  int Tp;              // T rounded up to a multiple of 32 (K-dimension of the aggregation)
  int NB;              // per-block state row: D*D entries of h^T then 2*D of z (hi, lo)
  int kc, kn, km;      // per-row counts (compute mode)
  float scale;         // softmax scale
  int mask_mode;
  bool global;         // linear branch over every key block (H_i, Z_i the same for all i)
  float gate;          // scale of the projected linear output (1 unless global)
  int G;               // two-level selection: key blocks per group (0: flat selection)
  int Tg, keep, ng;    // two-level selection: groups, kept groups, negligible groups per row
  long long BH() const { return static_cast<long long>(B) * H; }
};

// Byte offsets inside the caller's workspace.
struct WorkspaceLayout {
  size_t qbar, kbar;        // fp32 [BH, T, D]
  size_t kgbar;             // fp32 [BH, Tg, D]  group means of K (two-level selection)
  size_t scores;            // fp32 [BH, T, T]
  size_t lut, lut_cnt;      // int32 [BH, T, T] critical key blocks per row (ascending), int32 [BH, T]
  size_t col, col_cnt;      // int32 [BH, T, T] critical query blocks per column, int32 [BH, T]
  size_t rbits, cbits;      // uint32 [BH, Tp/32, Tp] marginal bits by row / by column, word-major:
                            // bit b of word w of row x is entry (x, 32 w + b)
  size_t states;            // bf16 [BH, Tp/4, NB, 4]  (forward h/z states; backward dH/dZ)
  size_t dstate;            // bf16 [BH, T, D*D] + fp32 [BH, T, 2, D] aggregated backward states
  size_t dstate_z;
  size_t dsum;              // fp32 [BH, N]  D_r of the backward
  size_t ddel;              // fp32 [BH, N]  linear-denominator gradient per row
  size_t dn;                // bf16 [BH, N, D]  dY / den per row
  size_t wT;                // bf16 [D, D]
  size_t dw_part;           // fp32 [P, D, D] dW partial sums
  size_t total;
};

struct SavedLayout {
  size_t lse, den, y, hst, zst, total;
};

constexpr int kDwParts = 512;
// runs of query blocks (one dW partial each) in the backward preparation
inline int dw_parts(const Dims& d) {
  const long long nblocks = d.BH() * d.T;
  return static_cast<int>(nblocks < kDwParts ? nblocks : kDwParts);
}

WorkspaceLayout workspace_layout(const Dims& d);
SavedLayout saved_layout(const Dims& d);

// ---- launchers (return hipSuccess or the launch error) ----
hipError_t launch_kv_state(const Dims& d, const uint16_t* k, const uint16_t* v, float* kbar,
                           uint16_t* states, hipStream_t s);
hipError_t launch_dstate(const Dims& d, const uint16_t* q, const uint16_t* dn, const float* ddel,
                         uint16_t* states, hipStream_t s);
hipError_t launch_pool(const Dims& d, const uint16_t* x, float* xbar, hipStream_t s);
hipError_t launch_scores(const Dims& d, const float* qbar, const float* kbar, float* scores,
                         hipStream_t s);
hipError_t launch_classify(const Dims& d, const float* scores, int8_t* mask, int32_t* lut,
                           int32_t* lut_cnt, uint32_t* rbits, hipStream_t s);
hipError_t launch_mask_lists(const Dims& d, const int8_t* mask, int32_t* lut, int32_t* lut_cnt,
                             uint32_t* rbits, int32_t* col, int32_t* col_cnt, uint32_t* cbits,
                             hipStream_t s);
hipError_t launch_fill_mask(const Dims& d, int8_t* mask, int8_t value, hipStream_t s);
// two-level selection: group means of K from the block means, the coarse score
// map alone, and the classification (from qbar / kgbar / kbar, or from given
// coarse and fine maps when coarse_in / scores_in are set)
hipError_t launch_group_means(const Dims& d, const float* kbar, float* kgbar, hipStream_t s);
hipError_t launch_coarse_scores(const Dims& d, const float* qbar, const float* kgbar,
                                float* coarse, hipStream_t s);
hipError_t launch_classify_hier(const Dims& d, const float* qbar, const float* kgbar,
                                const float* kbar, const float* coarse_in, const float* scores_in,
                                int8_t* mask, int32_t* lut, int32_t* lut_cnt, uint32_t* rbits,
                                hipStream_t s);
hipError_t launch_aggregate(const Dims& d, const uint32_t* bits, const uint16_t* states,
                            uint16_t* hout, float* zout, hipStream_t s);
// column sums of the states over every key block, written to slot i = 0 of
// each head of hout [BH, T, D*D] / zout [BH, T, 2D]
hipError_t launch_state_total(const Dims& d, const uint16_t* states, uint16_t* hout, float* zout,
                              hipStream_t s);
hipError_t launch_attn_fwd(const Dims& d, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* w, const int32_t* lut,
                           const int32_t* lut_cnt, bool dense, bool linear,
                           const uint16_t* hst, const float* zst, uint16_t* o, float* lse,
                           float* den, uint16_t* y, hipStream_t s);

// backward
hipError_t launch_w_transpose(const Dims& d, const uint16_t* w, uint16_t* wT, hipStream_t s);
hipError_t launch_bwd_prep(const Dims& d, const uint16_t* o, const uint16_t* dO,
                           const uint16_t* wT, const float* den, const uint16_t* y, bool linear,
                           float* dsum, float* ddel, uint16_t* dn, float* dw_part, hipStream_t s);
hipError_t launch_bwd_q(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dO, const float* lse, const float* dsum,
                        const int32_t* lut, const int32_t* lut_cnt, const uint16_t* dn,
                        const float* ddel, const uint16_t* hst, const float* zst, bool linear,
                        float* dq, hipStream_t s);
hipError_t launch_bwd_kv(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* lse, const float* dsum,
                         const int32_t* col, const int32_t* col_cnt, const uint16_t* dh,
                         const float* dz, bool linear, float* dk, float* dv, hipStream_t s);
hipError_t launch_dw_reduce(const Dims& d, const float* part, float* dw, hipStream_t s);

}  // namespace sla
