// Device-side helpers shared by the gfx950 kernels of the SLA library.
//
// MFMA operand layouts used throughout (wave64, bf16 inputs, fp32 accumulate):
//   v_mfma_f32_32x32x16_bf16: lane l holds A[m = l % 32][k = 8 (l / 32) + s] and
//     B[k = 8 (l / 32) + s][n = l % 32] for s = 0..7; result register i holds
//     C[m = 8 (i / 4) + 4 (l / 32) + i % 4][n = l % 32], i = 0..15.
//   v_mfma_f32_16x16x32_bf16: lane l holds A[m = l % 16][k = 8 (l / 16) + s],
//     B[k = 8 (l / 16) + s][n = l % 16]; result register i holds
//     C[m = 4 (l / 16) + i][n = l % 16], i = 0..3.
// Because an MFMA sums over k, any permutation of the k index that A and B
// share leaves the product unchanged; kernels use that to feed a 32x32 result
// tile straight back in as the B operand of the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
// Native vector types for register staging (HIP's uint4 class defeats
// scalar replacement of register arrays).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;
constexpr int kMaxT = 2048;   // most 64-token blocks per sequence (N <= 131072)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round-to-nearest-even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 8 fp32 -> bf16x8 operand (4 packed conversions).
__device__ __forceinline__ bf16x8 cvt_bf16x8(const float* x) {
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
  const u32x4_ w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// elu(x) + 1
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ float phi_prime(float x) { return x > 0.f ? 1.f : __expf(x); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}
__device__ __forceinline__ bf16x8 as_bf16x8(const uint2& lo, const uint2& hi) {
  uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return as_bf16x8(v);
}

// 16-bit element s (0..7) of a 16-byte register vector.
__device__ __forceinline__ uint32_t u4_elem(const u32x4& v, int s) {
  const uint32_t w = v[s >> 1];
  return (s & 1) ? (w >> 16) : (w & 0xffffu);
}
// 16-bit element s (0..3) of an 8-byte register vector.
__device__ __forceinline__ uint16_t u4_half(const u32x2& v, int s) {
  const uint32_t w = v[s >> 1];
  return static_cast<uint16_t>((s & 1) ? (w >> 16) : (w & 0xffffu));
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x2& lo, const u32x2& hi) {
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// A lane pair (l, l + 32) holding 8 consecutive bf16 of one row each, columns
// c0 + 8 hl .. + 7 (hl = l / 32), is turned into the two 4-column pieces the
// 32x32 MFMA result layout gives lane (row, hl) for that row: even = columns
// c0 + 4 hl .. + 3, odd = columns c0 + 8 + 4 hl .. + 3 (v_permlane32_swap
// exchanges the halves the other lane needs).
__device__ __forceinline__ void row_halves(const u32x4& x, u32x2& even, u32x2& odd) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  even = u32x2{s0[0], s1[0]};
  odd = u32x2{s0[1], s1[1]};
}
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte chunks addressed by
// lanes 4 s + i / 4 of its group, s = 0..3 (verified on the MI355X).  So when
// lane c of a group points at row kb + c / 4, column n0 + 4 (c % 4) of a
// row-major matrix, every lane gets M[kb + s][n0 + c], s = 0..3: four
// consecutive k values of its own column, i.e. a slice of an MFMA operand
// whose k index runs down the rows of the LDS tile.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Operand of v_mfma_f32_32x32x16 from a row-major LDS tile M[k][n] (pitch in
// elements, a multiple of 4): lane l gets M[r0 + s][n0 + l % 32] for the 8 k
// slots s, with row r0 + s for s < 4 and row r1 + s - 4 for s >= 4, where
// (r0, r1) = (kb + 8 h, kb + 8 h + 4) for natural k order, or
// (kb + 4 h, kb + 8 + 4 h) for the permuted order pi(h, s) that a 32x32 result
// tile has when it is reused as an operand (h = l / 32).
template <bool PERMUTED>
__device__ __forceinline__ bf16x8 lds_op32_tr(const uint16_t* m, int pitch, int kb, int n0,
                                              int lane) {
  const int g = lane >> 4, c = lane & 15, h = lane >> 5;
  const int col = n0 + 16 * (g & 1) + 4 * (c & 3);
  const int r0 = PERMUTED ? kb + 4 * h + (c >> 2) : kb + 8 * h + (c >> 2);
  const u32x2 lo = lds_tr4(m + r0 * pitch + col);
  const u32x2 hi = lds_tr4(m + (r0 + (PERMUTED ? 8 : 4)) * pitch + col);
  return as_bf16x8(lo, hi);
}

// Buffer resource over [base, base + bytes) (raw buffer, bounds-checked: reads
// past the end return zero) and a 16-byte load at voffset + soffset bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Workgroup id remapped so that consecutive logical ids share an XCD: the
// hardware deals workgroups round-robin over the 8 XCDs, each with its own L2.
// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): lane l of
// the wave writes its 16 bytes at lds_base + 16 l; lds_base must be uniform.
// Completion is tracked by vmcnt like any other vector load.
__device__ __forceinline__ void gl_to_lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(
      (__attribute__((address_space(1))) void*)(const_cast<void*>(gsrc)),
      (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// ---------------------------------------------------------------------------
// Unpadded row-major bf16 tiles in LDS (row length D) whose 16-byte chunks are
// XOR-swizzled per row: chunk k of row r sits in slot k ^ swz<D>(r).  Such a
// tile can be filled by the asynchronous global->LDS copy (which writes whole
// 1 KB runs), and both 16-byte row reads (16 lanes on 16 different rows) and
// transpose reads (4 rows x 32 bytes per 16 lanes) spread over the banks.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r))) << 3) + (col & 7);
}
// rows [0, rows) of a row-major global tile into a swizzled LDS tile; the
// calling workgroup's waves w = 0 .. nw-1 share the copies; completion is
// tracked by vmcnt
template <int D>
__device__ __forceinline__ void copy_swz(const uint16_t* src, uint16_t* dst, int rows, int w,
                                         int nw, int lane) {
  const int copies = rows * (D / 8) / 64;
  for (int it = w; it < copies; it += nw) {
    const int p = it * 64 + lane;
    const int r = p / (D / 8), sl = p % (D / 8);
    gl_to_lds16(src + r * D + 8 * (sl ^ swz<D>(r)), dst + it * 512);
  }
}
// lds_op32_tr<false> on a swizzled tile: lane gets M[kb + 8 (l/32) + s][n0 + l%32] (s < 4)
// and M[kb + 8 (l/32) + 4 + s][...] as the 32x32x16 operand layout
template <int D>
__device__ __forceinline__ bf16x8 swz_op32_tr(const uint16_t* m, int kb, int n0, int lane) {
  const int g = lane >> 4, c = lane & 15, h = lane >> 5;
  const int col = n0 + 16 * (g & 1) + 4 * (c & 3);
  const int r0 = kb + 8 * h + (c >> 2);
  return as_bf16x8(lds_tr4(m + swz_off<D>(r0, col)), lds_tr4(m + swz_off<D>(r0 + 4, col)));
}
// lds_op32_tr<true> (permuted k order) on a swizzled tile
template <int D>
__device__ __forceinline__ bf16x8 swz_op32_tr_perm(const uint16_t* m, int kb, int n0, int lane) {
  const int g = lane >> 4, c = lane & 15, h = lane >> 5;
  const int col = n0 + 16 * (g & 1) + 4 * (c & 3);
  const int r0 = kb + 4 * h + (c >> 2);
  return as_bf16x8(lds_tr4(m + swz_off<D>(r0, col)), lds_tr4(m + swz_off<D>(r0 + 8, col)));
}
// rows [row0, row0 + 64) of a row-major tile behind a buffer resource into a
// swizzled LDS tile (asynchronous buffer->LDS copies; bytes past the
// resource's size arrive as zero); the workgroup's waves share the copies
template <int D, int NW>
__device__ __forceinline__ void copy_swz_buf(__amdgpu_buffer_rsrc_t rs, int row0, uint16_t* dst,
                                             int w, int lane) {
  constexpr int kCopies = 64 * (D / 8) / 64;
  static_assert(kCopies % NW == 0, "copies split evenly over the waves");
#pragma unroll
  for (int u = 0; u < kCopies / NW; ++u) {
    const int it = w + NW * u;
    const int p = it * 64 + lane;
    const int r = p / (D / 8), sl = p % (D / 8);
    const int voff = ((row0 + r) * D + 8 * (sl ^ swz<D>(r))) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + it * 512),
                                             16, voff, 0, 0, 0);
  }
}
// Buffer resource over rows [row0, L) of a row-major bf16 matrix with D
// columns: copies through it read the padded rows at or past L as zero, and
// the row offset lives in the resource (scalar) instead of every lane's
// offset.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int row0, int L) {
  return make_rsrc(base + static_cast<size_t>(row0) * D,
                   static_cast<uint32_t>(L > row0 ? L - row0 : 0) * D * 2);
}
// Byte offset, within a 64-row tile, of this lane's 16 bytes in the u-th of
// the kCopies / NW copy instructions of wave w (the copy_swz_buf split); a
// per-lane constant.
template <int D, int NW>
__device__ __forceinline__ uint32_t swz_copy_voff(int w, int lane, int u) {
  const int it = w + NW * u;
  const int p = it * 64 + lane;
  const int r = p / (D / 8), sl = p % (D / 8);
  return static_cast<uint32_t>((r * D + 8 * (sl ^ swz<D>(r))) * 2);
}
// Copy instruction u of wave w into the swizzled LDS tile dst, from the
// rows of rs (built by rows_rsrc), with the lane offset voff from swz_copy_voff.
template <int D, int NW>
__device__ __forceinline__ void copy_swz_rows_one(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                  uint16_t* dst, int w, int u) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (w + NW * u) * 512),
                                           16, voff, 0, 0, 0);
}

// NaN-propagating maximum (IEEE 754-2019 maximum): v_maximum3_f32 on gfx950,
// with no canonicalisation of the inputs (fmaxf adds one per input)
__device__ __forceinline__ float fmax_p(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// maximum of the 16 elements of a result tile, three at a time
__device__ __forceinline__ float max16(const f32x16& v) {
  float m = fmax_p(fmax_p(v[0], v[1]), v[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) m = fmax_p(fmax_p(m, v[e]), v[e + 1]);
  return fmax_p(m, v[15]);
}
// four consecutive rows of one column: lane gets M[kb + 4 (l/32) + s][n0 + l%32], s < 4
template <int D>
__device__ __forceinline__ u32x2 swz_col4(const uint16_t* m, int kb, int n0, int lane) {
  const int g = lane >> 4, c = lane & 15, h = lane >> 5;
  const int col = n0 + 16 * (g & 1) + 4 * (c & 3);
  return lds_tr4(m + swz_off<D>(kb + 4 * h + (c >> 2), col));
}

__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t total) {
  if (total % 8u != 0u) return bid;
  return (bid % 8u) * (total / 8u) + bid / 8u;
}

}  // namespace sla
