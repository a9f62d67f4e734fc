// gfx950 (MI355X, CDNA4) kernels for sparse MLA decode with an index-driven
// KV gather.
//
// The method (FlashInfer "trtllm_batch_decode_sparse_mla_dsv4",
// introduction and parameters): each token's H query heads (512 dims) attend
// to the 512-d latent rows named by the token's row of a combined int32
// table (columns < 128: SWA pool, others: compressed pool, -1 masked,
// topk_lens truncating); every head shares the row as key and value; each
// head's softmax may include an attention-sink logit; the output is BF16
// plus a base-2 LSE (FlashInfer "cake_sparse_mla_sm120_dsv4_nvfp4_decode",
// parameters out_lse / lse_scale / attn_sink / mid_out / mid_lse).
//
// Kernel design (ours, for CDNA4; the pages' TRTLLM-gen / CuTe kernels are
// prior art only):
//  * One workgroup of 4 wave64s per (token, split), one wave per SIMD.  All H
//    heads of the token live in the workgroup, so each gathered row is read
//    from HBM once per (token, split) and reused by every head.
//  * The split's table columns are compacted first (masked, -1, truncated
//    and out-of-range slots are dropped), so tiles are dense.
//  * Rows are gathered 32 at a time (64 in decode_h64_kernel) into
//    row-major LDS tiles with a padded pitch (conflict-free row and
//    transposed reads), by LDS-DMA for BF16 rows and through registers for
//    FP8 rows and packed block-scaled rows
//    (widened to BF16 on the way; every E4M3FN value, and every E4M3FN value
//    times a power of two in BF16's normal range, is exactly a BF16 value).
//  * S^T = K Q^T on MFMA 32x32x16 BF16 (A = tile rows from LDS, B = 32
//    heads of Q held in registers).  The accumulator layout of S^T is the
//    B-operand layout P^T needs for O^T = V^T P^T, so probabilities go to
//    the second MFMA without a cross-lane shuffle; V^T comes from LDS with
//    transposing reads.
//  * Online softmax in base 2 against a reference max that is set by the
//    first tile and left alone; a tile exceeding it by more than 2^64 makes
//    the split start over with the higher reference, so O is never rescaled
//    and the result is exact up to rounding.
//  * decode_hd_kernel (H=128): wave w computes S for 32 heads but O for a
//    quarter of the output dims of all heads, with P exchanged through LDS
//    (see there).  decode_h64_kernel (H=64): the same split of O over four
//    waves, with S of a 64-row tile split over the waves by head block and
//    row block.  Head tiles (a plan choice at H=128) run an H=128 call on
//    decode_h64_kernel as 2T virtual tokens of 64 heads each.  FP8 q and FP8 rows are widened exactly to BF16 and
//    multiplied on the BF16 MFMA.
//  * Unsplit: the epilogue adds the sink and writes out / out_lse.  Split:
//    each split writes a BF16 partial and its base-2 LSE; a combine kernel
//    merges them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "internal.h"

namespace smla {
namespace {

constexpr int kD = kHeadDim;
constexpr int kTile = 32;          // rows per LDS tile
constexpr int kRowBytes = kD * 2;  // a BF16 row
// LDS row pitch: a BF16 row plus 48 B of padding (pitch = 48 mod 256).
// 16 lanes reading the same 16-B chunk of 16 consecutive rows then hit 16
// distinct 16-B bank groups, the 16 lanes of a transposed read (4 rows x 4
// 8-byte columns) hit disjoint banks, and every LDS address of the kernel is
// a per-lane base plus a compile-time immediate.
constexpr int kRowPitch = kRowBytes + 48;
constexpr int kTileBytes = kTile * kRowPitch;
constexpr float kLog2e = 1.4426950408889634f;
// A tile may exceed the running reference max by this much (base-2 logit
// units) before the split is restarted with a higher reference: with
// p <= 2^64 every probability and partial sum stays finite in BF16/FP32.
constexpr float kRefSlack = 64.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A compile-time bool as a value (selects variants of generic lambdas).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------

// 8 OCP E4M3FN bytes (two dwords) -> 8 BF16 values packed in four dwords,
// with the gfx950 conversion v_cvt_scalef32_pk_bf16_fp8 at scale 1.0: every
// E4M3FN value (bias 7, subnormals m * 2^-9, NaN at S.1111.111) is exactly
// a BF16 value, so the conversion is exact (checked against the bit-level
// decode for all 256 codes in every byte position).
__device__ __forceinline__ u32x4 widen_e4m3fn_x8(u32x2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true));
  return r;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two BF16 (round to nearest even) packed in one dword
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);    // v_log_f32 (base 2)
}

// max(v[i], v[i ^ 32]) on every lane, with one VALU lane swap (no LDS).
__device__ __forceinline__ float max_with_other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                                  __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (they complete in issue order).  Only vmcnt is constrained.
// S^T = K Q^T is issued from inline asm so that its 16-register accumulator
// lives in VGPRs while the compiler keeps the O^T accumulators (the PV
// builtin) in AGPRs: both products as builtins would need 272 accumulator
// registers of one kind.  The asm follows the MFMA hazard rules the
// compiler itself applies on gfx950: an MFMA may accumulate into the result
// of the previous MFMA of the same opcode back to back; an operand written
// by a VALU instruction needs 2 wait states before an MFMA reads it; a VALU
// read of an MFMA result needs the MFMA's passes plus a few wait states (18
// are inserted, more than the compiler's own 11).  The statements are not
// volatile, so LDS reads can still be scheduled ahead of them; their order
// follows the data dependence through the accumulator.
__device__ __forceinline__ f32x16 mfma_qk_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
      : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk_drain(f32x16& acc) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 1" : "+v"(acc));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One LDS-DMA row load: every lane fetches 16 bytes at `gaddr` and the
// hardware stores lane i's bytes at LDS byte address lds_addr + 16 i.  Issued
// from inline asm so that the compiler does not treat it as an LDS store it
// must wait for before every later LDS read (the pipeline below orders the
// tiles with explicit vmcnt waits and barriers).  M0 carries the LDS base;
// it is saved and restored around the load, which samples it at issue.
//
// The row address is wave-uniform: it lives in SGPRs (`row`) and each lane
// adds its own byte offset `lane_off` (16 * lane), so issuing a row costs
// scalar work only.
//
// STREAM: the load carries the non-temporal hint, for calls whose gathered
// rows are too many to still be cached when the next call runs (see
// kStreamingBytes below).
template <bool STREAM = false, bool ADDR_SETTLED = false>
__device__ __forceinline__ void lds_dma_row16(const uint8_t* row,
                                              uint32_t lane_off,
                                              uint32_t lds_addr) {
  uint32_t saved;
  // s_nop 4: the row address may have just been written by a VALU
  // (v_readlane / v_readfirstlane), and a VMEM read of a VALU-written SGPR
  // needs 5 wait states.  ADDR_SETTLED: the caller guarantees that more
  // than 5 instructions separate that write from this load (the steady
  // tile loop, whose row addresses are read out one iteration earlier).
  // s_nop 0: M0 written by SALU before LDS-DMA.
#define SMLA_DMA_BODY(NOP, NT)                     \
  asm volatile(NOP                                 \
               "s_mov_b32 %0, m0\n\t"              \
               "s_mov_b32 m0, %3\n\t"              \
               "s_nop 0\n\t"                       \
               "global_load_lds_dwordx4 %1, %2" NT "\n\t" \
               "s_mov_b32 m0, %0"                  \
               : "=&s"(saved)                      \
               : "v"(lane_off), "s"(row), "s"(lds_addr) \
               : "memory")
  if constexpr (STREAM && ADDR_SETTLED) SMLA_DMA_BODY("", " nt");
  else if constexpr (STREAM) SMLA_DMA_BODY("s_nop 4\n\t", " nt");
  else if constexpr (ADDR_SETTLED) SMLA_DMA_BODY("", "");
  else SMLA_DMA_BODY("s_nop 4\n\t", "");
#undef SMLA_DMA_BODY
}

// 8 bytes through a global (not flat) pointer (FP8 q: a per-lane head
// row): flat loads also count in lgkmcnt, which would make LDS waits wait
// for HBM too.
typedef u32x2 __attribute__((address_space(1))) global_u32x2;
__device__ __forceinline__ u32x2 load_global8(const uint8_t* row, uint32_t off) {
  return *(const global_u32x2*)(row + off);
}
typedef u32x4 __attribute__((address_space(1))) global_u32x4;
// 8 bytes per lane of a 512-byte FP8 row from a uniform row address: a
// buffer load with the row as a scalar resource and a 32-bit lane offset.
// The global form needs a 64-bit address per lane, built by the VALU for
// every row; this form measured 1.5-2.5% faster on FP8-row decodes, with
// the same bytes.  The resource covers exactly the row (offsets past it
// would read 0).
// Word 3 of the buffer resource: DATA_FORMAT (bits 18:15) = 4, 32-bit
// elements, which untyped loads need to be nonzero; no swizzle, no index
// stride, default destination selects.
constexpr int kRawBufferWord3 = 4 << 15;
__device__ __forceinline__ u32x2 load_row8(const uint8_t* row, uint32_t off) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, 512, kRawBufferWord3);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0));
}
typedef int32_t __attribute__((address_space(1))) global_i32;

// ---------------------------------------------------------------------------
// packed block-scaled FP8 rows (584 bytes)
// ---------------------------------------------------------------------------
//
// FlashInfer "trtllm_batch_decode_sparse_mla_dsv4" (introduction,
// packed-backend paragraph; parameter swa_kv_cache) gives the row's size,
// 584 bytes of uint8 per token, and vLLM DeepseekV4FlashInferMLAAttention
// (class comment on use_flashmla_fp8_layout) its family, UE8M0 block-scaled
// FP8.  The byte order is read as: NoPE dims 0..447 as E4M3FN codes (bytes
// 0..447), RoPE dims 448..511 as little-endian BF16 (bytes 448..575), then
// one UE8M0 scale byte per 56 NoPE dims (bytes 576..583); NoPE dim d is
// E4M3FN(byte d) * 2^(scale[d / 56] - 127).
//
// In the kernels every lane of a wave loads 16 bytes of a packed row in two
// 8-byte halves and writes 16 bytes of its BF16 LDS tile row at 16 lane:
//  * lane L < 56 loads the 8 NoPE codes of dims [8 L, 8 L + 8) and the 8
//    scale bytes, picks the scale of its block (L / 7) and writes the codes
//    widened with it (E4M3FN times a power of two is exactly a BF16 value in
//    the normal range);
//  * lane 56 + i loads the RoPE bytes [448 + 16 i, +16), which are BF16
//    already, and writes them as they are, to tile row bytes 896 + 16 i.
// So the store is one full-wave write per row, with no branch and no exec
// mask change.
constexpr int kPackedRowBytes = 584;
constexpr int kPackedNopeLanes = 56;       // lanes holding 8 NoPE codes each
constexpr int kPackedBlockLanes = 7;       // 56 dims per scale = 7 lanes
constexpr int kPackedScaleOff = 576;       // first scale byte in the row
constexpr int kPackedRopeOff = 448;        // first RoPE byte in the row
static_assert(kPackedNopeLanes * 16 == 2 * kPackedRopeOff,
              "the RoPE lanes' 16 lane bytes are the RoPE dims' tile offsets");

// The lane's two row byte offsets and its scale-byte selector.
struct PackedLane {
  uint32_t off_a, off_b;   // the two 8-byte halves
  uint32_t sel;            // v_perm selector: byte L / 7 of the scales, zeros above
  bool nope;               // the lane holds NoPE codes
};
__device__ __forceinline__ PackedLane packed_lane(int lane) {
  PackedLane pl;
  pl.nope = lane < kPackedNopeLanes;
  const uint32_t rope = kPackedRopeOff + 16u * (uint32_t)(lane - kPackedNopeLanes);
  pl.off_a = pl.nope ? 8u * (uint32_t)lane : rope;
  pl.off_b = pl.nope ? (uint32_t)kPackedScaleOff : rope + 8u;
  pl.sel = 0x0c0c0c00u | ((uint32_t)(lane / kPackedBlockLanes) & 7u);
  return pl;
}

// The lane's 16 bytes of a packed row, through a buffer resource that covers
// exactly the row.
__device__ __forceinline__ u32x4 packed_load_row(const uint8_t* row, const PackedLane& pl) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)row, (short)0, kPackedRowBytes, kRawBufferWord3);
  const u32x2 a = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)pl.off_a, 0, 0));
  const u32x2 b = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)pl.off_b, 0, 0));
  return u32x4{a[0], a[1], b[0], b[1]};
}

// UE8M0 scale byte e -> the scale operand of the scaled FP8 conversion.  The
// conversion reads only the exponent field of that operand, as an E8M0
// value (measured on gfx950: field 0 scales by 2^-127, field 255 gives NaN,
// as UE8M0 defines them), so the bits e << 23 are the whole decode; as a
// binary32 they would be 0 for e = 0 and +inf for e = 255, which is why the
// operand is not used as a number anywhere else.
__device__ __forceinline__ float ue8m0_scale(uint32_t e) {
  return __uint_as_float(e << 23);
}

// 8 E4M3FN codes times a power-of-two scale -> 8 BF16 values (exact for
// results in BF16's normal range).
__device__ __forceinline__ u32x4 widen_e4m3fn_x8_scaled(u32x2 v, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], scale, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], scale, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], scale, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], scale, true));
  return r;
}

// The 16 bytes the lane writes to its tile row at 16 lane: NoPE lanes
// their codes widened with the block's scale (byte sel of the scale bytes
// in v[2..3]), RoPE lanes the bytes as loaded.
__device__ __forceinline__ u32x4 packed_tile_bytes(u32x4 v, const PackedLane& pl) {
  const uint32_t e = __builtin_amdgcn_perm(v[3], v[2], pl.sel);
  const u32x4 w = widen_e4m3fn_x8_scaled(u32x2{v[0], v[1]}, ue8m0_scale(e));
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pl.nope ? w[i] : v[i];
  return r;
}

__device__ __forceinline__ void record_error(int32_t* err, int code, int t,
                                             int c) {
  if (atomicCAS(err, 0, code) == 0) {
    atomicExch(err + 1, t);
    atomicExch(err + 2, c);
  }
}

// A token's table as one row of columns [0, K): columns below P read the
// first table and name SWA rows, the others read the second table (at column
// c - P) and name compressed rows.  The combined form (FlashInfer
// trtllm_batch_decode_sparse_mla_dsv4, "sparse_indices"/"sparse_topk_lens":
// 128 SWA columns, one length counting both) and the two-segment form (same
// page, "swa_topk_lens"/"extra_sparse_indices"/"extra_sparse_topk_lens";
// the Cake page's "extra_indices"/"extra_topk_length": one length per
// table) differ only in where the tables and lengths come from.  In the
// page-table form (same page, HCA paragraph, "hca_compressed_block_tables")
// the second table holds page IDs and compressed slot j is row
// page[j / ps] * ps + j % ps.
//
// GEN = false is the combined form only (one row, 128 SWA columns, one
// length), compiled to a plain indexed load: the general view costs the
// kernels registers they do not have to spare.  KEEP = false forms the row
// address from the arguments at each load instead of keeping it (fewer live
// registers in the H=128 kernel; the H=64 kernel does better keeping it).
template <bool GEN, bool KEEP = true>
struct TokenTable {
  int t;
  const int32_t* row1;
  const int32_t* row2;
  int P;        // columns of the first table
  int ps;       // rows per page when the second table holds page IDs, else 0
  int L1, L2;   // active columns of each table
  // the stored entry of column c (whether or not the column is active); a
  // page-table row that does not fit an int comes back as -2 (invalid)
  __device__ __forceinline__ int raw(const DecodeParams& p, int c) const {
    if constexpr (!GEN && !KEEP)
      return *(const global_i32*)(p.indices + (int64_t)t * p.index_row_stride + c);
    if (GEN ? c < P : true) return *(const global_i32*)(row1 + c);
    const int j = c - P;
    if (ps == 0) return *(const global_i32*)(row2 + j);
    const int64_t r = (int64_t)*(const global_i32*)(row2 + j / ps) * ps + j % ps;
    return (r >= 0 && r <= 0x7FFFFFFF) ? (int)r : -2;
  }
  // column c is below its table's length (callers also keep c < end(),
  // which in the combined form already says so)
  __device__ __forceinline__ bool live(int c) const {
    if constexpr (!GEN) return true;
    return c < P ? c < L1 : c - P < L2;
  }
  // one past the last column that can be active
  __device__ __forceinline__ int end() const {
    if constexpr (!GEN) return L1;
    return L2 > 0 ? P + L2 : L1;
  }
  // column c names an SWA row
  __device__ __forceinline__ bool swa(int c) const {
    if constexpr (!GEN) return c < kSwaColumns;
    return c < P;
  }
};

template <bool GEN, bool KEEP = true>
__device__ __forceinline__ TokenTable<GEN, KEEP> token_table(const DecodeParams& p, int t) {
  TokenTable<GEN, KEEP> tt;
  tt.t = t;
  tt.row1 = (GEN || KEEP) ? p.indices + (int64_t)t * p.index_row_stride : nullptr;
  if constexpr (GEN) {
    tt.P = p.swa_cols;
    tt.row2 = p.indices2 + (int64_t)t * p.index_row_stride2;
    tt.ps = p.segmented == 2 ? p.page_size : 0;
  } else {
    tt.P = kSwaColumns;
    tt.row2 = nullptr;
    tt.ps = 0;
  }
  tt.L1 = tt.L2 = 0;
  return tt;
}

// The token's raw length(s), loaded early (they are used after the Q loads):
// combined form a = topk_len; two segments a, b = the two tables' lengths;
// page table a = window, b = window + compressed slots.
template <bool GEN>
__device__ __forceinline__ void token_length_loads(const DecodeParams& p, int t, int& a, int& b) {
  if constexpr (!GEN) {
    a = p.topk_lens ? p.topk_lens[t] : p.K;
    b = 0;
  } else {
    a = p.topk_lens ? p.topk_lens[t] : p.swa_cols;
    b = p.lens2 ? p.lens2[t] : (p.segmented == 2 ? p.swa_cols + p.K2 : p.K2);
  }
}

// Clamps the raw lengths into tt and reports whether they were in range.
// (Combined form: L1 is the whole length.)
template <bool GEN, bool KEEP>
__device__ __forceinline__ bool token_lengths(const DecodeParams& p, int a, int b,
                                              TokenTable<GEN, KEEP>& tt) {
  if constexpr (!GEN) {
    tt.L1 = min(max(a, 0), p.K);
    return a >= 0 && a <= p.K;
  }
  tt.L1 = min(max(a, 0), p.swa_cols);
  const int n = p.segmented == 2 ? b - tt.L1 : b;   // compressed slots
  tt.L2 = min(max(n, 0), p.K2);
  return a >= 0 && a <= p.swa_cols && n >= 0 && n <= p.K2;
}

// ---------------------------------------------------------------------------
// split kernel
// ---------------------------------------------------------------------------

// A 32x32x16 BF16 MFMA tile, as the hardware lays it out on a wave64:
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) .. +8)
//   B (16 x 32): lane l holds B[8*(l/32) .. +8)[l % 32]
//   C (32 x 32): lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l % 32]
// S^T = K Q^T puts tile rows on M and heads on N, so lane l owns head
// l % 32 and the rows 8a + 4*(l/32) + b (a, b in 0..3) of a 32-row tile.
// Read as the B operand of O^T = V^T P^T (K = rows), registers 8h .. 8h+7
// of that accumulator are exactly the k-slots of the h-th 16-row MFMA step
// when slot s of k-group kg stands for tile row 16h + 8*(s/4) + 4*kg + s%4.
// V^T is fetched in that row order with ds_read_b64_tr_b16, which hands
// output lane j of each 16-lane group element j%4 of the 8-byte words
// addressed by input lanes 4e + j/4 (e = 0..3).

__device__ __forceinline__ int tile_row_of_reg(int i, int kg) {
  return 8 * (i >> 2) + 4 * kg + (i & 3);
}

// The work item (token, split) a workgroup of 256 threads runs, XCD-aware:
// the hardware hands consecutive workgroup ids to the 8 XCDs round-robin,
// so each XCD gets a contiguous range of work items; the splits of one token
// and neighbouring tokens (which share rows in speculative decode) then run
// together on one XCD and share its L2.  XCD x owns the item range
// [lo, lo + cnt) and starts its workgroups in the order of blockIdx.x >> 3.
// With per-token lengths, and more items than CUs (the host sets
// rank_items; with one item per CU the order cannot matter and the ranking
// would only put a dependent load in front of every item's own loads), the
// items of the range are started longest first (rank by active columns of
// the item's split, ties by position): with one or two items per CU, taking
// them in token order lets the CUs that draw two long tokens set the end of
// a ragged batch (~9% at 512 tokens of topk_len uniform in [1024, 2048]);
// longest-first recovers it for ~0.5% on uniform batches.  Up to one item
// per thread; `lens` (cnt entries) and `pick` are LDS scratch, and every
// thread of the workgroup must call this.  head_shift: items count virtual
// tokens, token v >> head_shift of the table (head tiles).
template <bool GEN>
__device__ __forceinline__ int pick_item(const DecodeParams& p, int32_t* lens,
                                         int32_t* pick, int head_shift) {
  constexpr int NT = 256;
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int q8 = nblk >> 3, r8 = nblk & 7;
  const int lo = xcd * q8 + min(xcd, r8);
  int item = lo + (blockIdx.x >> 3);
  const int cnt = q8 + (xcd < r8 ? 1 : 0);
  const bool ragged = GEN ? (p.topk_lens != nullptr || p.lens2 != nullptr)
                          : p.topk_lens != nullptr;
  if (p.rank_items && ragged && cnt > 1 && cnt <= NT) {
    const int tid = threadIdx.x;
    int my_len = -1;
    if (tid < cnt) {
      // active columns of the item's split: [0, L1) and, for the general
      // table view, [P, P + L2), intersected with the split's columns
      const int vi = (lo + tid) / p.S, si = lo + tid - vi * p.S;
      const int ti = vi >> head_shift;
      int a, b;
      token_length_loads<GEN>(p, ti, a, b);
      TokenTable<GEN, false> ti_tab = token_table<GEN, false>(p, ti);
      token_lengths<GEN>(p, a, b, ti_tab);
      const int c0 = si * p.split_cols, c1 = c0 + p.split_cols;
      my_len = max(0, min(ti_tab.L1, c1) - c0);
      if constexpr (GEN)
        my_len += max(0, min(ti_tab.P + ti_tab.L2, c1) - max(ti_tab.P, c0));
      lens[tid] = my_len;
    }
    __syncthreads();
    if (tid < cnt) {
      int rank = 0;
      for (int k = 0; k < cnt; ++k) {
        const int lk = lens[k];
        rank += (lk > my_len || (lk == my_len && k < tid)) ? 1 : 0;
      }
      if (rank == (int)(blockIdx.x >> 3)) *pick = lo + tid;
    }
    __syncthreads();
    item = *pick;
    __syncthreads();   // the scratch is free again
  }
  return item;
}

// ---------------------------------------------------------------------------
// split kernel, H = 128 with BF16 rows: heads for S, output dims for O
// ---------------------------------------------------------------------------
//
// Four waves.  Wave w computes S^T and the softmax of heads [32w, 32w+32)
// (a 32 x 32 S^T tile per 32-row KV tile), but accumulates O^T
// for the output dims [128w, 128w+128) of all 128 heads.  P^T is exchanged
// through LDS in exactly the B-operand layout the O^T MFMAs take, so the
// exchange is one 16-byte store and one 16-byte load per lane and head
// block.  Each wave then reads only its quarter of every V tile with the
// (half-rate) transposing LDS reads.  O^T of tile i-1 is computed while the
// softmax of tile i runs on the VALU: the two are independent, so the
// exponentials fill the gaps between O^T MFMAs.
//
// With one wave per SIMD nothing else can issue MFMAs while a wave is busy
// elsewhere, so the per-row gather work is kept small: the compacted slot
// list is padded to whole tiles, a tile's row addresses are computed by
// one VALU pass (one row per lane) and read out into SGPRs, and each row
// costs one load instruction.

// KV_FP8: E4M3FN rows (or packed rows, PACKED) go through one register
// set, two tiles ahead, and are widened to BF16 as they are written to LDS;
// BF16 rows go by LDS-DMA.  GATHER_ONLY: the same compaction and BF16 row gather
// with no arithmetic and no output (a measurement aid: the attainable
// gather rate on the same tables).
// SERIAL (a check for LDS races, not a production path): every step of the
// tile pipeline completes, row loads included, and all waves meet at a
// barrier before the next step starts, so no two steps overlap.  The
// arithmetic is the same instruction for instruction, so a pipelined call
// must give the same bits; a difference exposes a race between the steps.
template <bool Q_FP8, bool KV_FP8, bool SPLIT, bool GATHER_ONLY = false, bool GEN = false,
          bool STREAM = false, bool PACKED = false, bool SERIAL = false>
__device__ __forceinline__ void decode_hd_body(const DecodeParams& p) {
  static_assert(!PACKED || (KV_FP8 && !Q_FP8), "packed rows: BF16 q, register-staged rows");
  auto serial_point = [](bool wait_loads) {
    if constexpr (SERIAL) {
      if (wait_loads) wait_vmcnt<0>();
      __syncthreads();
    }
  };
  constexpr int NW = 4, H = 128, NT = 256;
  constexpr int RPW = kTile / NW;         // rows each wave gathers per tile
  // LDS tiles: i-1 (read by O^T), i (S^T), i+1 and i+2 (landing).
  constexpr int NSTAGE = 4;
  constexpr int kSegHd = 2048;           // table columns per pass
  constexpr int CPT = kSegHd / NT;        // columns per thread in compaction
  constexpr int NHB = H / 32;             // head blocks
  constexpr int NDB = kD / NW / 32;       // 32-dim blocks of O per wave
  constexpr int kPBuf = NHB * 2 * 64;     // P^T of one tile, in u32x4
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[NSTAGE * kTileBytes];
  __shared__ __attribute__((aligned(16))) u32x4 p_lds[2 * kPBuf];
  // code of each active row of the segment (SWA: row, compressed: row with
  // bit 31 set), padded with the last active row up to a whole tile
  __shared__ __attribute__((aligned(16))) int32_t slots[kSegHd + 2 * kTile];
  __shared__ float inv_lds[H];
  __shared__ int32_t wave_cnt[NW];
  __shared__ int32_t restart_flag;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31;
  const int kg = lane >> 5;

  // the work item (see pick_item); slots[] is free until the compaction
  const int item = pick_item<GEN>(p, slots, slots + kSegHd, 0);
  const int t = item / p.S;
  const int s = item - t * p.S;
  const int head = wave * 32 + l32;       // head of this lane's S^T column

  // Loads in the order their results are needed: topk_len, the first
  // segment's table entries (fetched before topk_len is known; columns past
  // it are dropped in the compaction), then Q, all through global (not flat)
  // pointers so that LDS waits and barriers do not wait for them.  vmcnt
  // retires in order, so the compaction's wait for the table entries does
  // not wait for Q, and Q lands while the compaction runs.
  const int c_begin = s * p.split_cols;
  const int c_cap = min(p.K, c_begin + p.split_cols);
  TokenTable<GEN, false> tt = token_table<GEN, false>(p, t);
  int len_a, len_b;
  token_length_loads<GEN>(p, t, len_a, len_b);
  int rv[CPT];
  auto load_idx = [&](int seg0, int seg_hi) {
    const int cb = seg0 + threadIdx.x * CPT;
#pragma unroll
    for (int k = 0; k < CPT; ++k) rv[k] = (cb + k < seg_hi) ? tt.raw(p, cb + k) : -1;
  };
  load_idx(c_begin, min(c_cap, c_begin + kSegHd));
  __builtin_amdgcn_sched_barrier(0);

  bf16x8 qf[32];
  if constexpr (!GATHER_ONLY) {
    const size_t qrow = ((size_t)t * H + head) * kD;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) {
      const int d0 = kk * 16 + kg * 8;
      u32x4 v;
      if constexpr (Q_FP8)
        v = widen_e4m3fn_x8(load_global8((const uint8_t*)p.q + qrow, d0));
      else
        v = *(const global_u32x4*)((const uint16_t*)p.q + qrow + d0);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  const bool lens_ok = token_lengths<GEN>(p, len_a, len_b, tt);
  if (p.validate && threadIdx.x == 0 && s == 0 && !lens_ok) record_error(p.err, 2, t, -1);
  const int c_end = min(tt.end(), c_cap);

  float m_run = -INFINITY;
  float l_run = 0.f;
  // O^T: o[db][hb] holds dims 128w + 32db + 8(i/4) + 4kg + i%4 of head
  // 32hb + l32.
  f32x16 o[NDB][NHB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][hb][i] = 0.f;

  const int qk_off = l32 * kRowPitch + kg * 16;
  const int i16 = lane & 15, grp = lane >> 4;
  const int tr_off = (4 * (grp >> 1) + (i16 >> 2)) * kRowPitch +
                     (16 * (grp & 1) + 4 * (i16 & 3)) * 2 + wave * (NDB * 64);
  const uint32_t lane_off = (uint32_t)lane * 16u;

  if (threadIdx.x == 0) restart_flag = 0;
  bool need_sticky = false;

  constexpr int kLead = KV_FP8 ? 3 : 4;
  // `after_lead` runs once the first kLead operand reads are out (LDS reads
  // return in order, so reads issued there do not delay the first MFMA).
  auto qk = [&](const uint8_t* tb, auto&& every, auto&& after_lead) -> f32x16 {
    bf16x8 a[kLead];
#pragma unroll
    for (int k = 0; k < kLead; ++k) a[k] = *(const bf16x8*)(tb + qk_off + k * 32);
    after_lead();
    f32x16 acc;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) acc = mfma_qk_first(a[0], qf[0]);
      else mfma_qk(acc, a[kk % kLead], qf[kk]);
      if (kk + kLead < 32)
        a[kk % kLead] = *(const bf16x8*)(tb + qk_off + (kk + kLead) * 32);
      __builtin_amdgcn_sched_barrier(0);
      every(kk);
    }
    __builtin_amdgcn_sched_barrier(0);
    return acc;
  };

  // One step block: O^T += V^T P^T for the previous tile (DO_PV) with the
  // softmax of the current tile's S^T spread over its 32 MFMAs.  The
  // softmax writes P^T of the current tile to `pw`.  Rows past the end of a
  // ragged tile arrive with S^T = -inf and get probability 0.  Only one
  // instance of this block updates O, so O keeps one register assignment.
  // O^T operands from LDS: V^T fragment f = 4h + db (rows 16h.., dims
  // block db of this wave) and P^T fragment (h, hb).
  constexpr int kVLead = KV_FP8 ? 3 : 4;
  auto vfrag = [&](const uint8_t* vt, int f) -> bf16x8 {
    const uint8_t* vb = vt + tr_off + (16 * (f >> 2)) * kRowPitch + (f & 3) * 64;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3)))*)(vb));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3)))*)(vb + 8 * kRowPitch));
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pfrag = [&](const u32x4* pr, int h, int hb) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, pr[(hb * 2 + h) * 64 + lane]);
  };
  // The first O^T operands of a block are read before the S^T MFMAs that
  // precede it, so the block does not start with an LDS round trip.
  auto pv_prefetch = [&](const uint8_t* vt, const u32x4* pr, bf16x8 (&pfr)[NHB],
                         bf16x8 (&vfr)[kVLead]) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) pfr[hb] = pfrag(pr, 0, hb);
#pragma unroll
    for (int f = 0; f < kVLead; ++f) vfr[f] = vfrag(vt, f);
  };
  auto step_block = [&](auto do_pv, const uint8_t* vt, const u32x4* pr,
                        bf16x8 (&pfr)[NHB], bf16x8 (&vfr)[kVLead],
                        f32x16 sv, u32x4* pw, auto&& every) {
    constexpr bool kPV = decltype(do_pv)::value;
    // P^T operands of the second 16-row half: with a register set of their
    // own (kP1Early, BF16 rows) they are read eight MFMAs ahead of their
    // first use; otherwise (FP8 rows, which have no registers to spare)
    // P^T(1, hb) replaces P^T(0, hb) right after its last use, four MFMAs
    // before it is needed.
    constexpr bool kP1Early = !KV_FP8;
    float smax = 0.f, tmax = 0.f, lsum = 0.f, mx[5];
    bool need = false;
    u32x4 pk[2];
    bf16x8 pfr1[NHB];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kPV) {
        const int f = k >> 2, hb = k & 3;
        const bf16x8 pb = (kP1Early && f >= 4) ? pfr1[hb] : pfr[hb];
        o[f & 3][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vfr[f % kVLead], pb, o[f & 3][hb], 0, 0, 0);
        if (hb == 3 && f + kVLead < 8) vfr[f % kVLead] = vfrag(vt, f + kVLead);
        if constexpr (kP1Early) {
          if (f == 2) pfr1[hb] = pfrag(pr, 1, hb);
        } else {
          if (f == 3) pfr[hb] = pfrag(pr, 1, hb);
        }
      }
      // The softmax of the current tile, spread so that no step waits for
      // a result of the same MFMA slot: the max as a tree (k = 0, 1), the
      // reference max (k = 2, 3), then value j's logit at k = 3 + j, its
      // exponential at k = 4 + j, its sum and BF16 pair at k = 5 + j, and
      // P^T at k = 21.
      if (k == 0) {
        mx[0] = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
        mx[1] = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
        mx[2] = fmaxf(fmaxf(sv[6], sv[7]), sv[8]);
        mx[3] = fmaxf(fmaxf(sv[9], sv[10]), sv[11]);
        mx[4] = fmaxf(fmaxf(sv[12], sv[13]), sv[14]);
      } else if (k == 1) {
        smax = fmaxf(fmaxf(fmaxf(mx[0], mx[1]), sv[15]), fmaxf(fmaxf(mx[2], mx[3]), mx[4]));
        smax = max_with_other_half(smax);
      } else if (k == 2) {
        // The reference max is set by the first tile and then left alone,
        // so O is never rescaled inside the loop; a tile that outgrows it
        // by more than kRefSlack raises it and sets the sticky flag, and
        // the split restarts once with the raised reference (it only
        // grows, so one restart suffices).
        tmax = smax * p.scale_log2;     // scale_log2 > 0
        m_run = (m_run == -INFINITY) ? tmax : m_run;
        need = tmax > m_run + kRefSlack;
      }
      if (k == 3) {
        m_run = need ? tmax : m_run;
        need_sticky |= need;
      }
      if (k >= 3 && k < 19) {
        const int j = k - 3;
        sv[j] = __builtin_fmaf(sv[j], p.scale_log2, -m_run);
      }
      if (k >= 4 && k < 20) {
        const int j = k - 4;
        sv[j] = fast_exp2(sv[j]);
      }
      if (k >= 5 && k < 21) {
        const int j = k - 5;
        lsum += sv[j];
        if (j & 1) pk[j >> 3][(j & 7) >> 1] = pack_bf16x2(sv[j - 1], sv[j]);
      }
      if (k == 21) {
        pw[(wave * 2 + 0) * 64 + lane] = pk[0];
        pw[(wave * 2 + 1) * 64 + lane] = pk[1];
        l_run += lsum;
      }
      __builtin_amdgcn_sched_barrier(0);
      every(k);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto no_hook = [](int) {};

  bool again;
  bool first_seg = true;
  do {
  again = false;
  for (int seg0 = c_begin; seg0 < c_end && !again; seg0 += kSegHd) {
    const int seg1 = min(c_end, seg0 + kSegHd);

    // ---- compact the active slots of this segment into row addresses ------
    // Thread i takes CPT consecutive columns; all its index loads are in
    // flight together.  Slot order is column order.
    __syncthreads();   // the previous segment no longer reads slots[] / tiles
    if (!first_seg) {
      // Later segments (and restarts) reload the table and wait for it here,
      // where nothing else is in flight.  Without this wait the compiler
      // would have to wait for every load at the merge below, so the first
      // segment's compaction would also wait for all of Q.
      load_idx(seg0, seg1);
      wait_vmcnt<0>();
    }
    first_seg = false;
    const int cb = seg0 + threadIdx.x * CPT;
    uint32_t actm = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = cb + k;
      const int r = rv[k];
      if (r != -1 && c < seg1 && tt.live(c)) {
        const int64_t rows = tt.swa(c) ? p.swa_rows : p.comp_rows;
        if (r >= 0 && (int64_t)r < rows) actm |= 1u << k;
        else if (p.validate) record_error(p.err, 1, t, c);
      }
    }
    const int cnt = __popc(actm);
    // exclusive prefix of cnt (<= CPT < 16) over the wave: one ballot per
    // bit of cnt, each counted below this lane with mbcnt (no LDS trips)
    static_assert(CPT < 16, "four ballots cover cnt");
    int incl = cnt;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint64_t m = __ballot((cnt >> b) & 1);
      incl += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    }
    if (lane == 63) wave_cnt[wave] = incl;
    __syncthreads();
    int pos = incl - cnt, n_act = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const int cw = wave_cnt[w2];
      pos += (w2 < wave) ? cw : 0;
      n_act += cw;
    }
    int last = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if ((actm >> k) & 1u) {
        last = tt.swa(cb + k) ? rv[k] : (int)((uint32_t)rv[k] | 0x80000000u);
        slots[pos++] = last;
      }
    }
    // The owner of the last active slot pads the tail of the last tile.
    const int ntiles = (n_act + kTile - 1) / kTile;
    if (cnt > 0 && pos == n_act) {
      for (int i = n_act; i < ntiles * kTile; ++i) slots[i] = last;
    }
    __syncthreads();
    auto n_in = [&](int tile) { return min(kTile, n_act - tile * kTile); };
    auto stage = [&](int tile) -> const uint8_t* {
      return kv_lds + (tile % NSTAGE) * kTileBytes;
    };
    // The wave's RPW row addresses of a tile, in SGPRs: lane j converts
    // the code of row j on the VALU, then each address is read out of its
    // lane (a few instructions per tile instead of a scalar multiply chain
    // per row).
    // ... in three steps, so that the steady tile loop can spread them over
    // its MFMAs: the slot code (an LDS read), the lane's row address, and
    // the address of row jj read out of lane jj.
    auto row_code = [&](int tile) -> int {
      return slots[tile * kTile + wave_u * RPW + (lane & (RPW - 1))];
    };
    auto row_addr = [&](int code) -> uint64_t {
      const uint8_t* base = code < 0 ? p.comp : p.swa;
      return (uint64_t)(uintptr_t)(base + (int64_t)(code & 0x7FFFFFFF) * p.row_stride_bytes);
    };
    auto row_of_lane = [&](uint64_t a, int jj) -> const uint8_t* {
      // (readlane returns int: widen through uint32_t, not with sign
      // extension)
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a, jj);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), jj);
      return (const uint8_t*)(uintptr_t)((uint64_t)lo | ((uint64_t)hi << 32));
    };
    auto fetch_rows = [&](int tile, const uint8_t* (&rows)[RPW]) {
      const uint64_t a = row_addr(row_code(tile));
#pragma unroll
      for (int jj = 0; jj < RPW; ++jj) rows[jj] = row_of_lane(a, jj);
    };
    auto mask_tail = [&](f32x16& sv, int it) {
      const int nt = n_in(it);
      if (nt < kTile) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sv[i] = (tile_row_of_reg(i, kg) < nt) ? sv[i] : -INFINITY;
      }
    };

    const uint32_t lds_base = (uint32_t)(uintptr_t)kv_lds;
    auto issue_row = [&](int tile, int jj, const uint8_t* row) {
      const uint32_t dst = lds_base + (uint32_t)((tile % NSTAGE) * kTileBytes) +
                           (uint32_t)((wave_u * RPW + jj) * kRowPitch);
      lds_dma_row16<STREAM>(row, lane_off, dst);
    };
    // The same, from a tile base computed once (the wave's first row of the
    // tile's stage), with row addresses read out an iteration earlier.
    auto issue_row_settled = [&](uint32_t tile_base, int jj, const uint8_t* row) {
      lds_dma_row16<STREAM, true>(row, lane_off, tile_base + (uint32_t)(jj * kRowPitch));
    };
    // The first row gathers go out without waiting for Q: loads retire in
    // order, so the wait for tile 0 also covers Q.  (The compiler's own
    // waits for the last Q fragments, which count only its loads, may then
    // also wait for some of tile 1's rows in the first S^T: a one-off cost
    // far below Q's latency.)

    if constexpr (KV_FP8) {
      if (ntiles > 0) {
        // FP8 rows: each lane loads 8 bytes of each of the wave's 8 rows.
        // One register set: inside the S^T MFMAs of tile it, row jj of tile
        // it+1 is widened from it and written to LDS, and then row jj of
        // tile it+2 is loaded into it, so every load has about one tile of
        // MFMA work to land.  These are ordinary loads, so the compiler's
        // own waits are exact.
        std::conditional_t<PACKED, u32x4, u32x2> rs[RPW];
        const uint8_t* rows[RPW];
        const uint32_t lane_off8 = (uint32_t)lane * 8u;
        const PackedLane pl = packed_lane(lane);   // packed rows only
        // one row of `tile` into its registers
        auto load_one = [&](int tile, int jj) {
          if constexpr (PACKED) rs[jj] = packed_load_row(rows[jj], pl);
          else rs[jj] = load_row8(rows[jj], lane_off8);
        };
        auto store_one = [&](int tile, int jj) {
          uint8_t* dst = kv_lds + (tile % NSTAGE) * kTileBytes +
                         (wave_u * RPW + jj) * kRowPitch;
          if constexpr (PACKED)
            *(u32x4*)(dst + lane * 16) = packed_tile_bytes(rs[jj], pl);
          else
            *(u32x4*)(dst + lane * 16) = widen_e4m3fn_x8(rs[jj]);
        };
        fetch_rows(0, rows);
#pragma unroll
        for (int jj = 0; jj < RPW; ++jj) load_one(0, jj);
#pragma unroll
        for (int jj = 0; jj < RPW; ++jj) store_one(0, jj);
        fetch_rows(min(1, ntiles - 1), rows);
#pragma unroll
        for (int jj = 0; jj < RPW; ++jj) load_one(1, jj);
        fetch_rows(min(2, ntiles - 1), rows);
        // One iteration.  QK: tile it exists; MOVE: store tile it+1 and load
        // tile it+2.  Both are compile-time so that the loop body has no
        // branches and the compiler's load waits stay exact (at a branch
        // merge it would wait for every load).  Rows past the last tile
        // re-read valid rows (fetch_rows clamps), which hit in L2, and are
        // stored to a stage that no S^T reads.
        auto iteration = [&](auto pv, auto qk_on, auto move_on, int it) {
          constexpr bool kQK = decltype(qk_on)::value;
          constexpr bool kMove = decltype(move_on)::value;
          // tile it is in LDS, P^T of tile it-1 is written, and the readers
          // of the previous iteration are done
          __syncthreads();
          const u32x4* pr = p_lds + ((it + 1) & 1) * kPBuf;      // tile it-1
          const uint8_t* vt = kv_lds + ((it + NSTAGE - 1) % NSTAGE) * kTileBytes;
          f32x16 sv;
          // The first O^T operands of tile it-1 are read inside the S^T
          // MFMAs (P^T after MFMAs 16..19, V^T after 24, 26, 28).
          bf16x8 pfr[NHB], vfr[kVLead];
          if constexpr (kQK) {
            sv = qk(stage(it), [&](int kk) {
              if (kMove && (kk & 3) == 1) store_one(it + 1, kk >> 2);
              if (kMove && (kk & 3) == 3) load_one(it + 2, kk >> 2);
              if constexpr (decltype(pv)::value) {
                if (kk >= 16 && kk < 16 + NHB) pfr[kk - 16] = pfrag(pr, 0, kk - 16);
                if (kk >= 24 && kk < 24 + 2 * kVLead && ((kk - 24) & 1) == 0)
                  vfr[(kk - 24) >> 1] = vfrag(vt, (kk - 24) >> 1);
              }
            }, [] {});
            mfma_qk_drain(sv);
            mask_tail(sv, it);
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = -INFINITY;   // no tile: P = 0
            if constexpr (decltype(pv)::value) pv_prefetch(vt, pr, pfr, vfr);
          }
          serial_point(true);
          // the row addresses of tile it+3 (those of tile it+2 were used by
          // the loads above): slot code under the first MFMAs, readouts
          // between the last ones, which have no softmax work beside them
          int code = 0;
          uint64_t addr = 0;
          step_block(pv, vt, pr, pfr, vfr, sv, p_lds + (it & 1) * kPBuf, [&](int k) {
            if constexpr (kMove) {
              if (k == 4) code = row_code(min(it + 3, ntiles - 1));
              if (k == 23) addr = row_addr(code);
              if (k >= 24 && k < 24 + RPW) rows[k - 24] = row_of_lane(addr, k - 24);
            }
          });
          serial_point(false);
        };
        using T_ = BoolC<true>;
        using F_ = BoolC<false>;
        // the first tile (with one tile only, its moves fill an unused
        // stage), every later tile but the last, the last, and the drain
        iteration(F_{}, T_{}, T_{}, 0);
        int it = 1;
        for (; it + 1 < ntiles; ++it) iteration(T_{}, T_{}, T_{}, it);
        if (ntiles > 1) iteration(T_{}, T_{}, F_{}, ntiles - 1);
        iteration(T_{}, F_{}, F_{}, ntiles);
      }
    } else if (ntiles > 0) {
      // LDS-DMA gather, two tiles ahead.
      const uint8_t* rows[RPW];
      for (int tl = 0; tl < min(2, ntiles); ++tl) {
        fetch_rows(tl, rows);
#pragma unroll
        for (int jj = 0; jj < RPW; ++jj) issue_row(tl, jj, rows[jj]);
      }
      fetch_rows(min(2, ntiles - 1), rows);
      // The RPW rows of tile it+2 go out during the S^T MFMAs of tile it.
      auto qk_tile = [&](int it, bool do_issue) -> f32x16 {
        if constexpr (GATHER_ONLY) {
          f32x16 none;
#pragma unroll
          for (int i = 0; i < 16; ++i) none[i] = -INFINITY;
          if (do_issue) {
#pragma unroll
            for (int jj = 0; jj < RPW; ++jj) issue_row(it + 2, jj, rows[jj]);
          }
          return none;
        }
        f32x16 sv = qk(stage(it), [&](int kk) {
          if (do_issue && (kk & 3) == 3) issue_row(it + 2, kk >> 2, rows[kk >> 2]);
        }, [] {});
        mfma_qk_drain(sv);
        mask_tail(sv, it);
        return sv;
      };
      // Wait until this wave's rows of tile it landed (the rows of tile
      // it+1 may still be in flight), then for every wave's: the barrier
      // also orders P^T of tile it-1 before its readers and frees the stage
      // of tile it-2 for tile it+2.
      auto land = [&](int it) {
        if (!SERIAL && it + 1 < ntiles) wait_vmcnt<RPW>();
        else wait_vmcnt<0>();
        __syncthreads();
      };
      land(0);
      {
        const bool di = 2 < ntiles;
        bf16x8 pfr[NHB], vfr[kVLead];
        const f32x16 sv0 = qk_tile(0, di);
        serial_point(true);
        if constexpr (!GATHER_ONLY)
          step_block(BoolC<false>{}, kv_lds, p_lds, pfr, vfr, sv0, p_lds, no_hook);
        if (di) fetch_rows(min(3, ntiles - 1), rows);
        serial_point(false);
      }
      // Iteration it: land tile it, O^T of tile it-1 with the S^T and
      // softmax of tile it, the rows of tile it+2 issued during S^T.  STEADY
      // iterations (it + 2 < ntiles) are a compile-time variant: every row
      // issue happens and tile it is whole, so the body has no branches.
      auto iteration = [&](auto steady, int it) {
        constexpr bool kSteady = decltype(steady)::value && !GATHER_ONLY;
        if constexpr (kSteady) {
          if constexpr (SERIAL) wait_vmcnt<0>();
          else wait_vmcnt<RPW>();
          __syncthreads();
        } else {
          if (it < ntiles) land(it);
          else __syncthreads();
        }
        const bool di = kSteady || it + 2 < ntiles;
        const u32x4* pr = p_lds + ((it - 1) & 1) * kPBuf;
        bf16x8 pfr[NHB], vfr[kVLead];
        f32x16 sv;
        if constexpr (kSteady) {
          // The first O^T operands are read inside the S^T MFMAs, spread
          // out (P^T after MFMAs 8..11, V^T after MFMAs 20, 22, 24, 26):
          // read before the S^T chain they held 32 registers across it, and
          // their LDS trips sat between the first S^T operand reads.
          const uint32_t tile_base = lds_base + (uint32_t)(((it + 2) % NSTAGE) * kTileBytes) +
                                     (uint32_t)(wave_u * RPW * kRowPitch);
          const uint8_t* vt = stage(it - 1);
          sv = qk(stage(it), [&](int kk) {
            if ((kk & 3) == 3) issue_row_settled(tile_base, kk >> 2, rows[kk >> 2]);
            if (kk >= 8 && kk < 8 + NHB) pfr[kk - 8] = pfrag(pr, 0, kk - 8);
            if (kk >= 20 && kk < 20 + 2 * kVLead && (kk & 1) == 0)
              vfr[(kk - 20) >> 1] = vfrag(vt, (kk - 20) >> 1);
          }, [] {});
          mfma_qk_drain(sv);
        } else if (it < ntiles) {
          if constexpr (!GATHER_ONLY) pv_prefetch(stage(it - 1), pr, pfr, vfr);
          sv = qk_tile(it, di);
        } else {
          if constexpr (!GATHER_ONLY) pv_prefetch(stage(it - 1), pr, pfr, vfr);
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[i] = -INFINITY;   // no tile: P = 0
        }
        serial_point(true);
        if constexpr (kSteady) {
          // The rows of tile it+3 (their addresses are no longer needed for
          // tile it+2, whose loads went out above): the slot code is read
          // under the first O^T MFMAs, the readouts into SGPRs go between the
          // last ones, which have no softmax work beside them.
          int code = 0;
          uint64_t addr = 0;
          step_block(BoolC<true>{}, stage(it - 1), pr, pfr, vfr, sv,
                     p_lds + (it & 1) * kPBuf, [&](int k) {
                       if (k == 4) code = row_code(min(it + 3, ntiles - 1));
                       if (k == 23) addr = row_addr(code);
                       if (k >= 24 && k < 24 + RPW) rows[k - 24] = row_of_lane(addr, k - 24);
                     });
        } else {
          if constexpr (!GATHER_ONLY)
            step_block(BoolC<true>{}, stage(it - 1), pr, pfr, vfr, sv,
                       p_lds + (it & 1) * kPBuf, no_hook);
          if (di) fetch_rows(min(it + 3, ntiles - 1), rows);
        }
        serial_point(false);
      };
      int it = 1;
      for (; it + 2 < ntiles; ++it) iteration(BoolC<true>{}, it);
      for (; it <= ntiles; ++it) iteration(BoolC<false>{}, it);
    }
    if (__ballot(need_sticky) != 0ull && lane == 0) restart_flag = 1;
    __syncthreads();
    again = restart_flag != 0;
  }
  if (again) {
    // Rare: start the split over with the raised reference maxima.
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) restart_flag = 0;
    need_sticky = false;
    l_run = 0.f;
    // A zero made here (opaque to the compiler): a plain 0.f would be
    // merged with the initial clearing of O, and the compiler would then
    // keep a block of zero registers alive across the whole tile loop
    // (spilled to scratch by every workgroup).
    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][hb][i] = zero;
  }
  } while (again);
  if constexpr (GATHER_ONLY) return;
  // ---- epilogue: the head owner finishes its head's normaliser ------------
  {
    float l = l_run + __shfl_xor(l_run, 32);
    float m = m_run;
    float inv, lse;
    if constexpr (SPLIT) {
      inv = (l > 0.f) ? p.bmm2 / l : 0.f;
      lse = (l > 0.f) ? m + fast_log2(l) : -INFINITY;
    } else {
      float fac = 1.f;
      if (p.sinks) {
        const float sl = p.sinks[head] * kLog2e;
        const float mm = fmaxf(m, sl);
        fac = fast_exp2(m - mm);       // 0 when nothing was active (m = -inf)
        l = l * fac + fast_exp2(sl - mm);
        m = mm;
      }
      inv = (l > 0.f) ? fac * p.bmm2 / l : 0.f;
      lse = (l > 0.f) ? p.lse_scale * (m + fast_log2(l)) : -INFINITY;
    }
    if (kg == 0) {
      inv_lds[head] = inv;
      if constexpr (SPLIT) p.mid_lse[((size_t)t * H + head) * p.S + s] = lse;
      else if (p.out_lse) p.out_lse[(size_t)t * H + head] = lse;
    }
  }
  __syncthreads();
  // ---- O goes out through LDS as whole 1 KB head rows ---------------------
  // (the tiles are no longer in use).  Two passes of 64 heads: every wave
  // writes its 128 dims of each head, then each wave stores whole rows.
  constexpr int kOutPitch = kD * 2 + 16;
  static_assert(64 * kOutPitch <= NSTAGE * kTileBytes, "epilogue staging");
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const int hb = 2 * pass + hq;
      const float inv = inv_lds[hb * 32 + l32];
      uint8_t* rowp = kv_lds + (hq * 32 + l32) * kOutPitch + wave * (NDB * 64) + kg * 8;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][hb][4 * a] * inv, o[db][hb][4 * a + 1] * inv);
          w[1] = pack_bf16x2(o[db][hb][4 * a + 2] * inv, o[db][hb][4 * a + 3] * inv);
          *(u32x2*)(rowp + db * 64 + a * 16) = w;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r * NW + wave;
      const int hh = pass * 64 + row;
      const u32x4 v = *(const u32x4*)(kv_lds + row * kOutPitch + lane * 16);
      uint16_t* dst;
      if constexpr (SPLIT)
        dst = p.mid_out + (((size_t)t * H + hh) * p.S + s) * kD;
      else
        dst = (uint16_t*)p.out + ((size_t)t * H + hh) * kD;
      *(u32x4*)(dst + lane * 8) = v;
    }
    if (pass == 0) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// split kernel, H = 64: four waves, 64-row tiles
// ---------------------------------------------------------------------------
//
// One workgroup of four waves fills the CU: wave w computes S^T and the
// softmax of heads [32(w&1), +32) over rows [32(w>>1), +32) of a 64-row
// tile, and O^T for the output dims [128w, +128) of all 64 heads over all 64
// rows, with P^T exchanged through LDS in the O^T MFMAs' B-operand layout
// (as in decode_hd_kernel).  (Two workgroups of two waves, each wave
// holding 32 heads of O for all 512 dims, would make every wave read the
// whole tile for both products: a third more LDS reads per row.)
// Two LDS stages of 64 rows: the rows of tile i+1 go out during the S^T
// MFMAs of tile i, by LDS-DMA (BF16 rows) or into registers (FP8 and
// packed rows; widened and written to their stage between the O^T MFMAs of
// tile i, the stage tile i-1 used).  The two waves that share a head block
// share its reference max: the first tile's is the max over both row
// blocks (exchanged through LDS), and a restart takes the larger of the
// two waves' raised maxima.  The normaliser adds the two waves' sums.
template <bool Q_FP8, bool KV_FP8, bool SPLIT, bool GEN, bool PACKED = false,
          bool SERIAL = false>
__global__ __launch_bounds__(256, 1)
void decode_h64_kernel(DecodeParams p) {
  static_assert(!PACKED || (KV_FP8 && !Q_FP8), "packed rows: BF16 q, register-staged rows");
  static_assert(!Q_FP8 || KV_FP8, "FP8 q needs FP8 rows");
  constexpr int NW = 4, H = 64, NT = 256;
  constexpr int TR = 64;                  // tile rows
  constexpr int RPW = TR / NW;            // rows each wave gathers per tile
  constexpr int NSTAGE = 2;
  constexpr int kSegHd = 2048;            // table columns per pass
  constexpr int CPT = kSegHd / NT;        // columns per thread in compaction
  constexpr int NDB = kD / NW / 32;       // 32-dim blocks of O per wave
  constexpr int NHB = H / 32;             // head blocks
  constexpr int NKS = TR / 16;            // 16-row steps of O^T
  constexpr int kStageBytes = TR * kRowPitch;
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[NSTAGE * kStageBytes];
  __shared__ __attribute__((aligned(16))) u32x4 p_lds[NHB * NKS * 64];
  __shared__ __attribute__((aligned(16))) int32_t slots[kSegHd + TR];
  __shared__ float inv_lds[H];
  __shared__ float pair_lds[2][H];        // per row block: a head's max, then its sum
  __shared__ int32_t wave_cnt[NW];
  __shared__ int32_t restart_flag;
  auto serial_point = [](bool wait_loads) {
    if constexpr (SERIAL) {
      if (wait_loads) wait_vmcnt<0>();
      __syncthreads();
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31;
  const int kg = lane >> 5;
  const int hbs = wave & 1, rbs = wave >> 1;   // this wave's S^T block
  const int head = hbs * 32 + l32;             // head of this lane's S^T column

  // the work item (see pick_item); slots[] is free until the compaction.
  // With head tiles (an H=128 call) item v of the grid is virtual token
  // vt: table token t = vt >> 1, heads hoff + 0..63; q, the output and the
  // partials are indexed by vt, in the H=128 layout seen as 64 heads.
  const int item = pick_item<GEN>(p, slots, slots + kSegHd, p.head_shift);
  const int vt = item / p.S;
  const int s = item - vt * p.S;
  const int t = vt >> p.head_shift;
  const int hoff = (vt & ((1 << p.head_shift) - 1)) * H;

  // table entries, then Q (see decode_hd_kernel)
  const int c_begin = s * p.split_cols;
  const int c_cap = min(p.K, c_begin + p.split_cols);
  TokenTable<GEN, false> tt = token_table<GEN, false>(p, t);
  int len_a, len_b;
  token_length_loads<GEN>(p, t, len_a, len_b);
  int rv[CPT];
  auto load_idx = [&](int seg0, int seg_hi) {
    const int cb = seg0 + threadIdx.x * CPT;
#pragma unroll
    for (int k = 0; k < CPT; ++k) rv[k] = (cb + k < seg_hi) ? tt.raw(p, cb + k) : -1;
  };
  load_idx(c_begin, min(c_cap, c_begin + kSegHd));
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 qf[32];
  {
    const size_t qrow = ((size_t)vt * H + head) * kD;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) {
      const int d0 = kk * 16 + kg * 8;
      u32x4 v;
      if constexpr (Q_FP8)
        v = widen_e4m3fn_x8(load_global8((const uint8_t*)p.q + qrow, d0));
      else
        v = *(const global_u32x4*)((const uint16_t*)p.q + qrow + d0);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const bool lens_ok = token_lengths<GEN>(p, len_a, len_b, tt);
  if (p.validate && threadIdx.x == 0 && s == 0 && !lens_ok) record_error(p.err, 2, t, -1);
  const int c_end = min(tt.end(), c_cap);

  float m_run = -INFINITY;
  float l_run = 0.f;
  bool ref_set = false;
  // O^T: o[db][hb] holds dims 128w + 32db + 8(i/4) + 4kg + i%4 of head
  // 32hb + l32.
  f32x16 o[NDB][NHB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][hb][i] = 0.f;

  const int qk_off = (rbs * 32 + l32) * kRowPitch + kg * 16;
  const int i16 = lane & 15, grp = lane >> 4;
  const int tr_off = (4 * (grp >> 1) + (i16 >> 2)) * kRowPitch +
                     (16 * (grp & 1) + 4 * (i16 & 3)) * 2 + wave * (NDB * 64);
  const uint32_t lane_off = (uint32_t)lane * 16u;
  const uint32_t lds_base = (uint32_t)(uintptr_t)kv_lds;
  if (threadIdx.x == 0) restart_flag = 0;
  bool need_sticky = false;

  // S^T of this wave's 32 rows of the tile at tb; every4(q) after MFMA 4q+3
  constexpr int kLead = 4;
  auto qk = [&](const uint8_t* tb, auto&& every4) -> f32x16 {
    bf16x8 a[kLead];
#pragma unroll
    for (int k = 0; k < kLead; ++k) a[k] = *(const bf16x8*)(tb + qk_off + k * 32);
    f32x16 acc;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) acc = mfma_qk_first(a[0], qf[0]);
      else mfma_qk(acc, a[kk % kLead], qf[kk]);
      if (kk + kLead < 32)
        a[kk % kLead] = *(const bf16x8*)(tb + qk_off + (kk + kLead) * 32);
      if ((kk & 3) == 3) {
        __builtin_amdgcn_sched_barrier(0);
        every4(kk >> 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    return acc;
  };
  auto vfrag = [&](const uint8_t* vt, int f) -> bf16x8 {
    const uint8_t* vb = vt + tr_off + (16 * (f >> 2)) * kRowPitch + (f & 3) * 64;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3)))*)(vb));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3)))*)(vb + 8 * kRowPitch));
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pfrag = [&](int h, int hb) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, p_lds[(hb * NKS + h) * 64 + lane]);
  };
  // O^T += V^T P^T over the tile's 64 rows.  MFMA k: 16-row step h = k/8,
  // dim block db = (k/2) % 4, head block hb = k % 2; V^T fragment f = 4h + db
  // is read two fragments ahead, P^T of step h+1 during step h.  hook(k)
  // runs after MFMA k.
  auto ot = [&](const uint8_t* vt, auto&& hook) {
    bf16x8 v[3], pf[2][NHB];
    pf[0][0] = pfrag(0, 0);
    pf[0][1] = pfrag(0, 1);
    v[0] = vfrag(vt, 0);
    v[1] = vfrag(vt, 1);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      __builtin_amdgcn_sched_barrier(0);
      const int h = k >> 3, db = (k >> 1) & 3, hb = k & 1, f = 4 * h + db;
      o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[f % 3], pf[h & 1][hb],
                                                         o[db][hb], 0, 0, 0);
      if (hb == 1 && f + 2 < 4 * NKS) v[(f + 2) % 3] = vfrag(vt, f + 2);
      if ((k & 7) == 3 && h + 1 < NKS) {
        pf[(h + 1) & 1][0] = pfrag(h + 1, 0);
        pf[(h + 1) & 1][1] = pfrag(h + 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      hook(k);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // The softmax of this wave's 32 rows of a tile with nt valid rows (rows
  // past nt get probability 0), P^T to LDS.
  auto softmax_pt = [&](f32x16 sv, int nt) {
    if (nt < TR) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sv[i] = (rbs * 32 + tile_row_of_reg(i, kg) < nt) ? sv[i] : -INFINITY;
    }
    float smax = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) smax = fmaxf(fmaxf(smax, sv[i]), sv[i + 1]);
    smax = max_with_other_half(fmaxf(smax, sv[15]));
    float tmax = smax * p.scale_log2;          // scale_log2 > 0
    if (!ref_set) {
      // the first tile: the reference is the max over both row blocks
      if (kg == 0) pair_lds[rbs][head] = tmax;
      __syncthreads();
      m_run = fmaxf(pair_lds[0][head], pair_lds[1][head]);
      ref_set = true;
    }
    const bool need = tmax > m_run + kRefSlack;
    m_run = need ? tmax : m_run;
    need_sticky |= need;
    float lsum = 0.f;
    u32x4 pk[2];
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(sv[j], p.scale_log2, -m_run));
      const float p1 = fast_exp2(__builtin_fmaf(sv[j + 1], p.scale_log2, -m_run));
      lsum += p0 + p1;
      pk[j >> 3][(j & 7) >> 1] = pack_bf16x2(p0, p1);
    }
    l_run += lsum;
    p_lds[(hbs * NKS + 2 * rbs + 0) * 64 + lane] = pk[0];
    p_lds[(hbs * NKS + 2 * rbs + 1) * 64 + lane] = pk[1];
  };
  auto no_hook = [](int) {};

  bool again;
  bool first_seg = true;
  do {
  again = false;
  for (int seg0 = c_begin; seg0 < c_end && !again; seg0 += kSegHd) {
    const int seg1 = min(c_end, seg0 + kSegHd);

    // ---- compact the active slots of this segment (see decode_hd_kernel) --
    __syncthreads();
    if (!first_seg) {
      load_idx(seg0, seg1);
      wait_vmcnt<0>();
    }
    first_seg = false;
    const int cb = seg0 + threadIdx.x * CPT;
    uint32_t actm = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = cb + k;
      const int r = rv[k];
      if (r != -1 && c < seg1 && tt.live(c)) {
        const int64_t rows = tt.swa(c) ? p.swa_rows : p.comp_rows;
        if (r >= 0 && (int64_t)r < rows) actm |= 1u << k;
        else if (p.validate) record_error(p.err, 1, t, c);
      }
    }
    const int cnt = __popc(actm);
    static_assert(CPT < 16, "four ballots cover cnt");
    int incl = cnt;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint64_t m = __ballot((cnt >> b) & 1);
      incl += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    }
    if (lane == 63) wave_cnt[wave] = incl;
    __syncthreads();
    int pos = incl - cnt, n_act = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const int cw = wave_cnt[w2];
      pos += (w2 < wave) ? cw : 0;
      n_act += cw;
    }
    int last = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if ((actm >> k) & 1u) {
        last = tt.swa(cb + k) ? rv[k] : (int)((uint32_t)rv[k] | 0x80000000u);
        slots[pos++] = last;
      }
    }
    const int ntiles = (n_act + TR - 1) / TR;
    if (cnt > 0 && pos == n_act) {
      for (int i = n_act; i < ntiles * TR; ++i) slots[i] = last;
    }
    __syncthreads();
    auto stage = [&](int tile) -> const uint8_t* {
      return kv_lds + (tile % NSTAGE) * kStageBytes;
    };
    if constexpr (!KV_FP8) {
    if (ntiles > 0) {
      // lane j < RPW: the address of this wave's row j of `tile`
      auto lane_row_addr = [&](int tile) -> uint64_t {
        const int code = slots[tile * TR + wave_u * RPW + (lane & (RPW - 1))];
        const uint8_t* base = code < 0 ? p.comp : p.swa;
        return (uint64_t)(uintptr_t)(base + (int64_t)(code & 0x7FFFFFFF) * p.row_stride_bytes);
      };
      auto row_of_lane = [&](uint64_t a, int jj) -> const uint8_t* {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a, jj);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), jj);
        return (const uint8_t*)(uintptr_t)((uint64_t)lo | ((uint64_t)hi << 32));
      };
      auto tile_lds = [&](int tile) -> uint32_t {
        return lds_base + (uint32_t)((tile % NSTAGE) * kStageBytes) +
               (uint32_t)(wave_u * RPW * kRowPitch);
      };
      {
        const uint64_t a0 = lane_row_addr(0);
#pragma unroll
        for (int jj = 0; jj < RPW; ++jj)
          lds_dma_row16(row_of_lane(a0, jj), lane_off, tile_lds(0) + (uint32_t)(jj * kRowPitch));
      }
      for (int it = 0; it < ntiles; ++it) {
        wait_vmcnt<0>();                // this wave's rows of tile it landed
        __syncthreads();                // every wave's; O^T of tile it-1 done
        const bool more = it + 1 < ntiles;
        // the rows of tile it+1 go out during the S^T MFMAs, two per four
        // MFMAs, each read out at the hook before
        const uint64_t an = lane_row_addr(more ? it + 1 : it);
        const uint32_t dn = tile_lds(it + 1);
        constexpr int PER = RPW / 8;
        const uint8_t* rr[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) rr[r] = row_of_lane(an, r);
        f32x16 sv = qk(stage(it), [&](int q) {
          if (more) {
#pragma unroll
            for (int r = 0; r < PER; ++r)
              lds_dma_row16<false, true>(rr[r], lane_off,
                                         dn + (uint32_t)((q * PER + r) * kRowPitch));
          }
          if (q + 1 < 8) {
#pragma unroll
            for (int r = 0; r < PER; ++r) rr[r] = row_of_lane(an, (q + 1) * PER + r);
          }
        });
        mfma_qk_drain(sv);
        serial_point(true);
        softmax_pt(sv, min(TR, n_act - it * TR));
        __syncthreads();                // P^T of tile it published
        ot(stage(it), no_hook);
        serial_point(false);
      }
    }
    } else {
    if (ntiles > 0) {
      // FP8 and packed rows through registers: each lane holds 8 bytes of
      // an FP8 row (16 of a packed row) for each of the wave's RPW rows of
      // the next tile.  Row addresses come from a scalar chain per row
      // (with the loads' registers live, reading one VALU pass out per row
      // costs more than it saves).  These are ordinary loads, so the compiler's
      // own waits before the stores are exact.
      typedef std::conditional_t<PACKED, u32x4, u32x2> stage_t;
      stage_t st[RPW];
      const uint32_t lane_off8 = (uint32_t)lane * 8u;
      const PackedLane pl = packed_lane(lane);   // packed rows only
      // the slot codes of rows jj, jj+1 of this wave's rows of `tile`
      auto fetch_codes = [&](int tile, int jj) -> u32x2 {
        return *(const u32x2*)(slots + tile * TR + wave_u * RPW + jj);
      };
      auto load_row = [&](int jj, uint32_t raw) {
        const int code = __builtin_amdgcn_readfirstlane((int)raw);
        const uint8_t* base = code < 0 ? p.comp : p.swa;
        const uint8_t* row = base + (int64_t)(code & 0x7FFFFFFF) * p.row_stride_bytes;
        if constexpr (PACKED) st[jj] = packed_load_row(row, pl);
        else st[jj] = load_row8(row, lane_off8);
      };
      auto store_row = [&](int tile, int jj) {
        uint8_t* dst = kv_lds + (tile % NSTAGE) * kStageBytes +
                       (wave_u * RPW + jj) * kRowPitch + lane * 16;
        if constexpr (PACKED) *(u32x4*)dst = packed_tile_bytes(st[jj], pl);
        else *(u32x4*)dst = widen_e4m3fn_x8(st[jj]);
      };
      {
#pragma unroll
        for (int jj = 0; jj < RPW; jj += 2) {
          const u32x2 c = fetch_codes(0, jj);
          load_row(jj, c[0]);
          load_row(jj + 1, c[1]);
        }
#pragma unroll
        for (int jj = 0; jj < RPW; ++jj) store_row(0, jj);
      }
      // STEADY iterations (a next tile exists) are a compile-time variant,
      // so that no branch sits between the loads and their stores (at a
      // branch merge the compiler would wait for every load).
      auto iteration = [&](auto steady, int it) {
        constexpr bool kSteady = decltype(steady)::value;
        __syncthreads();                // tile it stored by every wave; O^T of it-1 done
        // two rows per four S^T MFMAs, their codes read at the hook before
        static_assert(RPW == 16, "two rows per hook");
        u32x2 codes = {0u, 0u};
        if constexpr (kSteady) codes = fetch_codes(it + 1, 0);
        f32x16 sv = qk(stage(it), [&](int q) {
          if constexpr (kSteady) {
            load_row(2 * q, codes[0]);
            load_row(2 * q + 1, codes[1]);
            if (q + 1 < 8) codes = fetch_codes(it + 1, 2 * q + 2);
          }
        });
        mfma_qk_drain(sv);
        serial_point(true);
        softmax_pt(sv, min(TR, n_act - it * TR));
        __syncthreads();                // P^T of tile it published
        // the next tile's rows go to its stage (free since the first
        // barrier), one row per two O^T MFMAs
        static_assert(2 * RPW <= 32, "a row per two O^T MFMAs");
        ot(stage(it), [&](int k) {
          if constexpr (kSteady) {
            if ((k & 1) == 0 && (k >> 1) < RPW) store_row(it + 1, k >> 1);
          }
        });
        serial_point(false);
      };
      int it = 0;
      for (; it + 1 < ntiles; ++it) iteration(BoolC<true>{}, it);
      iteration(BoolC<false>{}, it);
    }
    }
    if (__ballot(need_sticky) != 0ull && lane == 0) restart_flag = 1;
    __syncthreads();
    again = restart_flag != 0;
  }
  if (again) {
    // Rare: start the split over with the raised reference maxima, the same
    // for the two waves of a head block.
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) restart_flag = 0;
    if (kg == 0) pair_lds[rbs][head] = m_run;
    __syncthreads();
    m_run = fmaxf(pair_lds[0][head], pair_lds[1][head]);
    need_sticky = false;
    l_run = 0.f;
    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][hb][i] = zero;
  }
  } while (again);

  // ---- epilogue -------------------------------------------------------------
  // A head's sum: this wave's 32 rows (both halves of the wave), plus the
  // other row block's.
  __syncthreads();                      // pair_lds is free
  {
    const float lb = l_run + __shfl_xor(l_run, 32);
    if (kg == 0) pair_lds[rbs][head] = lb;
  }
  __syncthreads();
  if (rbs == 0) {
    float l = pair_lds[0][head] + pair_lds[1][head];
    float m = m_run;
    float inv, lse;
    if constexpr (SPLIT) {
      inv = (l > 0.f) ? p.bmm2 / l : 0.f;
      lse = (l > 0.f) ? m + fast_log2(l) : -INFINITY;
    } else {
      float fac = 1.f;
      if (p.sinks) {
        const float sl = p.sinks[hoff + head] * kLog2e;
        const float mm = fmaxf(m, sl);
        fac = fast_exp2(m - mm);        // 0 when nothing was active (m = -inf)
        l = l * fac + fast_exp2(sl - mm);
        m = mm;
      }
      inv = (l > 0.f) ? fac * p.bmm2 / l : 0.f;
      lse = (l > 0.f) ? p.lse_scale * (m + fast_log2(l)) : -INFINITY;
    }
    if (kg == 0) {
      inv_lds[head] = inv;
      if constexpr (SPLIT) p.mid_lse[((size_t)vt * H + head) * p.S + s] = lse;
      else if (p.out_lse) p.out_lse[(size_t)vt * H + head] = lse;
    }
  }
  __syncthreads();
  // O goes out through LDS as whole 1 KB head rows (the tiles are no longer
  // in use): every wave writes its 128 dims of each head, then each wave
  // stores whole rows.
  constexpr int kOutPitch = kD * 2 + 16;
  static_assert(H * kOutPitch <= NSTAGE * kStageBytes, "epilogue staging");
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float inv = inv_lds[hb * 32 + l32];
    uint8_t* rowp = kv_lds + (hb * 32 + l32) * kOutPitch + wave * (NDB * 64) + kg * 8;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][hb][4 * a] * inv, o[db][hb][4 * a + 1] * inv);
        w[1] = pack_bf16x2(o[db][hb][4 * a + 2] * inv, o[db][hb][4 * a + 3] * inv);
        *(u32x2*)(rowp + db * 64 + a * 16) = w;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < H / NW; ++r) {
    const int hh = r * NW + wave;
    const u32x4 v = *(const u32x4*)(kv_lds + hh * kOutPitch + lane * 16);
    uint16_t* dst;
    if constexpr (SPLIT)
      dst = p.mid_out + (((size_t)vt * H + hh) * p.S + s) * kD;
    else
      dst = (uint16_t*)p.out + ((size_t)vt * H + hh) * kD;
    *(u32x4*)(dst + lane * 8) = v;
  }
}

template <bool Q_FP8, bool KV_FP8, bool SPLIT, bool GEN, bool STREAM, bool PACKED = false,
          bool SERIAL = false>
__global__ __launch_bounds__(256, 1)
void decode_hd_kernel(DecodeParams p) {
  decode_hd_body<Q_FP8, KV_FP8, SPLIT, false, GEN, STREAM, PACKED, SERIAL>(p);
}

// The row gather of decode_hd_kernel alone (BF16 rows), under its own name.
template <bool STREAM>
__global__ __launch_bounds__(256, 1)
void gather_only_kernel(DecodeParams p) {
  decode_hd_body<false, false, false, true, false, STREAM>(p);
}

// ---------------------------------------------------------------------------
// combine kernel: one wave per (token, head); lane owns 8 output dims
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256)
void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  // The same XCD-aware mapping as the split kernels: XCD x takes the x-th
  // contiguous range of blocks, i.e. about the same tokens whose partials
  // it wrote, so they are read from its own L2.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int q8 = nblk >> 3, r8 = nblk & 7;
  const int blk = xcd * q8 + min(xcd, r8) + (blockIdx.x >> 3);
  const int item = blk * 4 + (threadIdx.x >> 6);
  if (item >= p.T * p.H) return;
  const int h = item % p.H;
  const float* ml = p.mid_lse + (size_t)item * p.stride;
  const uint16_t* base = p.mid_out + (size_t)item * p.stride * kD + lane * 8;
  // Every load goes out before any result is used, so the memory latencies
  // of the LSEs, the sink and the first kFirst partial rows overlap.  An
  // empty split's weight is 0 (its partial row is 0 too), so it is read and
  // added like any other.
  constexpr int kFirst = 16, kBatch = 8;
  const float mine = (lane < p.S) ? ml[lane] : -INFINITY;
  // (loaded without a branch; with no sinks the value read is unused)
  const float sink = *(p.sinks ? p.sinks + h : ml);
  u32x4 v[kFirst];
#pragma unroll
  for (int j = 0; j < kFirst; ++j)
    if (j < p.S) v[j] = *(const u32x4*)(base + (size_t)j * kD);

  float L = wave_max(mine);
  const float sl = p.sinks ? sink * kLog2e : -INFINITY;
  L = fmaxf(L, sl);
  float w = 0.f;
  if (lane < p.S && mine != -INFINITY) w = fast_exp2(mine - L);
  float W = wave_sum(w);
  if (p.sinks) W += fast_exp2(sl - L);

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  auto add = [&](const u32x4& row, float ws) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += ws * __uint_as_float(row[i] << 16);
      acc[2 * i + 1] += ws * __uint_as_float(row[i] & 0xFFFF0000u);
    }
  };
#pragma unroll
  for (int j = 0; j < kFirst; ++j)
    if (j < p.S) add(v[j], __shfl(w, j));
  for (int s0 = kFirst; s0 < p.S; s0 += kBatch) {
    u32x4 vb[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < p.S) vb[j] = *(const u32x4*)(base + (size_t)(s0 + j) * kD);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < p.S) add(vb[j], __shfl(w, s0 + j));
  }
  const float inv = (W > 0.f) ? 1.f / W : 0.f;
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *(u32x4*)(p.out + (size_t)item * kD + lane * 8) = r;
  if (lane == 0 && p.out_lse)
    p.out_lse[item] = (W > 0.f) ? p.lse_scale * (L + fast_log2(W)) : -INFINITY;
}

// ---------------------------------------------------------------------------
// combined-table builder: four output columns per thread
// ---------------------------------------------------------------------------
//
// The step before the decode (vLLM DeepseekV4FlashInferMLAAttention,
// _build_sparse_index_metadata): token t's row of the combined table is its
// SWA row followed by its compressed entries, a request-local position p
// becoming row block_tables[req][p / page_size] * page_size + p % page_size
// (the canonical page expansion of FlashInfer's hca_sparse_indices_format)
// and a global row being copied.  Columns past the token's compressed
// length are -1, its length is W + that length; a padding token (or one
// whose request index is out of range) gets an all -1 row and length 0.
// An entry that cannot be translated becomes -1 and is recorded in err.

constexpr int kBuildCols = 4;   // columns per thread, 256 apart (coalesced)

__global__ __launch_bounds__(256)
void build_indices_kernel(BuildParams p) {
  const int K = p.W + p.K2;
  const int per_row = (K + 256 * kBuildCols - 1) / (256 * kBuildCols);
  const int t = blockIdx.x / per_row;
  const int c0 = (blockIdx.x - t * per_row) * (256 * kBuildCols) + threadIdx.x;
  // the token's flags and length and this thread's entries are independent
  // loads, issued together; only the block-table lookups depend on them
  const int valid_raw = p.valid ? p.valid[t] : 1;
  const int req = p.token_to_req ? p.token_to_req[t] : t;
  const int len_raw = p.comp_lens ? p.comp_lens[t] : p.K2;
  int e[kBuildCols];
#pragma unroll
  for (int k = 0; k < kBuildCols; ++k) {
    const int c = c0 + 256 * k;
    e[k] = -1;
    if (c < p.W) e[k] = p.swa[(int64_t)t * p.swa_stride + c];
    else if (c < K) e[k] = p.comp[(int64_t)t * p.comp_stride + (c - p.W)];
  }
  bool valid = valid_raw != 0;
  if (valid && p.local && (req < 0 || req >= p.num_requests)) {
    valid = false;
    if (p.err && c0 == 0) record_error(p.err, 1, t, -1);
  }
  const int n2 = min(max(len_raw, 0), p.K2);
  if (c0 == 0) p.out_lens[t] = valid ? p.W + n2 : 0;
#pragma unroll
  for (int k = 0; k < kBuildCols; ++k) {
    const int c = c0 + 256 * k;
    if (c >= K) break;
    int v = -1;
    if (valid) {
      if (c < p.W) {
        v = e[k];
      } else if (c - p.W < n2 && e[k] >= 0) {
        if (!p.local) {
          v = e[k];
        } else {
          const int blk = e[k] / p.page_size;
          bool bad = blk >= p.max_blocks;
          if (!bad) {
            const int page = p.block_tables[(int64_t)req * p.bt_stride + blk];
            const int64_t row = (int64_t)page * p.page_size + e[k] % p.page_size;
            bad = page < 0 || row > 0x7FFFFFFF;
            if (!bad) v = (int)row;
          }
          if (bad && p.err) record_error(p.err, 1, t, c);
        }
      }
    }
    p.out[(int64_t)t * p.out_stride + c] = v;
  }
}

__global__ void clear_error_kernel(int32_t* err) {
  if (threadIdx.x < 4) err[threadIdx.x] = (threadIdx.x == 0) ? 0 : -1;
}

// Streaming rows.  A call that can gather at least this many bytes of BF16
// rows (T x K x 1 KB) does not leave them in MI355X's 256 MB last-level
// cache (Infinity Cache) for the next call, so its LDS-DMA row loads carry
// the non-temporal hint.  Measured at H=128, K=2048 against the plain loads:
// T=512 (1 GB) 3-4% faster, T=128 (256 MB) 1.5-2.5% faster, T=64 (128 MB)
// 1.5% slower and K=512 at T=64 (32 MB) 5% slower, where back-to-back calls
// on the same tables still find their rows cached.
constexpr int64_t kStreamingBytes = int64_t(256) << 20;

bool streaming_rows(const DecodeParams& p) {
  return (int64_t)p.T * p.K * (kHeadDim * 2) >= kStreamingBytes;
}

// GEN: the two-segment and page-table forms; the combined form runs the
// plain table view.
template <bool QF, bool KF, bool STREAM>
hipError_t launch_decode_hd_s(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.T * p.S));
  const bool gen = p.segmented != 0;
  if (p.serial) {            // combined table only (checked on the host)
    if (gen) return hipErrorInvalidValue;
    if (p.S > 1)
      hipLaunchKernelGGL((decode_hd_kernel<QF, KF, true, false, false, false, true>), grid,
                         dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_hd_kernel<QF, KF, false, false, false, false, true>), grid,
                         dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (p.S > 1 && gen)
    hipLaunchKernelGGL((decode_hd_kernel<QF, KF, true, true, STREAM>), grid, dim3(256), 0, stream, p);
  else if (p.S > 1)
    hipLaunchKernelGGL((decode_hd_kernel<QF, KF, true, false, STREAM>), grid, dim3(256), 0, stream, p);
  else if (gen)
    hipLaunchKernelGGL((decode_hd_kernel<QF, KF, false, true, STREAM>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_hd_kernel<QF, KF, false, false, STREAM>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// FP8 rows go through registers (no LDS-DMA), so only BF16 rows stream.
template <bool QF, bool KF>
hipError_t launch_decode_hd(const DecodeParams& p, hipStream_t stream) {
  if constexpr (!KF) {
    if (streaming_rows(p) && !p.serial) return launch_decode_hd_s<QF, KF, true>(p, stream);
  }
  return launch_decode_hd_s<QF, KF, false>(p, stream);
}

// Packed block-scaled FP8 rows (BF16 q), H = 128.
hipError_t launch_decode_hd_packed(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.T * p.S));
  const bool gen = p.segmented != 0;
  if (p.serial) {
    if (gen) return hipErrorInvalidValue;
    if (p.S > 1)
      hipLaunchKernelGGL((decode_hd_kernel<false, true, true, false, false, true, true>), grid,
                         dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_hd_kernel<false, true, false, false, false, true, true>), grid,
                         dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (p.S > 1 && gen)
    hipLaunchKernelGGL((decode_hd_kernel<false, true, true, true, false, true>), grid, dim3(256), 0, stream, p);
  else if (p.S > 1)
    hipLaunchKernelGGL((decode_hd_kernel<false, true, true, false, false, true>), grid, dim3(256), 0, stream, p);
  else if (gen)
    hipLaunchKernelGGL((decode_hd_kernel<false, true, false, true, false, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_hd_kernel<false, true, false, false, false, true>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// H = 64: the four-wave kernel.
template <bool QF, bool KF, bool PK = false>
hipError_t launch_decode_h64(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.T * p.S));
  const bool gen = p.segmented != 0;
  if (p.serial) {            // combined table only (checked on the host)
    if (gen) return hipErrorInvalidValue;
    if (p.S > 1)
      hipLaunchKernelGGL((decode_h64_kernel<QF, KF, true, false, PK, true>), grid, dim3(256), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((decode_h64_kernel<QF, KF, false, false, PK, true>), grid, dim3(256), 0,
                         stream, p);
    return hipGetLastError();
  }
  if (p.S > 1 && gen)
    hipLaunchKernelGGL((decode_h64_kernel<QF, KF, true, true, PK>), grid, dim3(256), 0, stream, p);
  else if (p.S > 1)
    hipLaunchKernelGGL((decode_h64_kernel<QF, KF, true, false, PK>), grid, dim3(256), 0, stream, p);
  else if (gen)
    hipLaunchKernelGGL((decode_h64_kernel<QF, KF, false, true, PK>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_h64_kernel<QF, KF, false, false, PK>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scratch of the allocation-free decode
// ---------------------------------------------------------------------------
//
// sparse_mla_decode_noalloc serves callers that cannot allocate device
// memory: its split partials (mid_lse, mid_out) and error block live in this
// array instead of a caller workspace.  Each GPU the library runs on holds
// its own copy (kNoAllocScratchBytes) from the module's load until the
// process ends.  Calls on one GPU share it, so calls that overlap on one GPU
// race; the partials are fully written by the split kernel before the
// combine reads them, so nothing in it has to start at zero.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept: in host code the array's name
// is only a host-side stand-in and must never be passed to a kernel.
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int q_dtype, int kv_dtype,
                         hipStream_t stream) {
  if (kv_dtype == kKvPacked584) {        // BF16 q only (checked on the host)
    if (q_dtype != 0) return hipErrorInvalidValue;
    if (p.H == 64) return launch_decode_h64<false, true, true>(p, stream);
    return launch_decode_hd_packed(p, stream);
  }
  const bool qf = q_dtype != 0, kf = kv_dtype != 0;
  if (p.H == 64) {
    if (!qf && !kf) return launch_decode_h64<false, false>(p, stream);
    if (qf && kf) return launch_decode_h64<true, true>(p, stream);
    return launch_decode_h64<false, true>(p, stream);
  }
  if (!kf) return launch_decode_hd<false, false>(p, stream);   // Q FP8 needs FP8 rows
  if (qf) return launch_decode_hd<true, true>(p, stream);
  return launch_decode_hd<false, true>(p, stream);
}

hipError_t launch_gather_only(const DecodeParams& p, hipStream_t stream) {
  if (p.H != 128) return hipErrorInvalidValue;
  if (streaming_rows(p))
    hipLaunchKernelGGL(gather_only_kernel<true>, dim3((unsigned)(p.T * p.S)),
                       dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(gather_only_kernel<false>, dim3((unsigned)(p.T * p.S)),
                       dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int items = p.T * p.H;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_clear_error(int32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(clear_error_kernel, dim3(1), dim3(64), 0, stream, err);
  return hipGetLastError();
}

hipError_t launch_build_indices(const BuildParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.T * ((p.W + p.K2 + 256 * kBuildCols - 1) / (256 * kBuildCols));
  hipLaunchKernelGGL(build_indices_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla
