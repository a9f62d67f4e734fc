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
//  * One workgroup of 4 wave64s per (token, split).  All H heads of the
//    token live in the workgroup, so each gathered row is read from HBM
//    once per (token, split) and reused by every head.  Wave w owns heads
//    [w*H/4, (w+1)*H/4): 16 heads (H=64) or 32 heads (H=128).
//  * The split's table columns are compacted in LDS first (masked, -1,
//    truncated and out-of-range slots are dropped), so tiles are dense.
//  * Rows are gathered 32 at a time into a double-buffered, XOR-swizzled
//    row-major LDS tile (FP8 rows are widened to BF16 on the way; every
//    E4M3FN value is exactly a BF16 value).
//  * S^T = K * Q^T on MFMA 16x16x32 BF16 (A = tile rows from LDS, B = the
//    wave's Q held in registers).  The accumulator layout of S^T puts one
//    head per lane column, which is exactly the B-operand layout P^T needs
//    for O^T = V^T * P^T, so softmax probabilities go to the second MFMA
//    without any cross-lane shuffle.
//  * Online softmax in base 2 with a lazily refreshed running max (the
//    reference max only moves when a tile's max exceeds it by more than 8,
//    so O is rarely rescaled); the final normalisation uses the same
//    reference, so the result is exact up to rounding.
//  * Unsplit: the epilogue adds the sink and writes out / out_lse.  Split:
//    each split writes a BF16 partial and its base-2 LSE; a combine kernel
//    merges them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace smla {
namespace {

constexpr int kD = kHeadDim;
constexpr int kTile = 32;          // rows per LDS tile
constexpr int kThreads = 256;      // 4 wave64
constexpr int kSeg = 2048;         // table columns compacted per pass
constexpr int kRowBytes = kD * 2;  // a BF16 row
// LDS row pitch: a BF16 row plus 16 B of padding.  Consecutive rows then
// start 4 banks apart, so 16 lanes reading the same 16-B chunk of 16
// consecutive rows hit distinct banks, and every LDS address of the kernel
// is a per-lane base plus a compile-time immediate.
constexpr int kRowPitch = kRowBytes + 16;
constexpr int kTileBytes = kTile * kRowPitch;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------

// OCP E4M3FN byte -> BF16 bits, exact (bias 7, subnormals m * 2^-9, NaN at
// S.1111.111).  A BF16 value keeps 8 significant bits, E4M3FN at most 4.
__device__ __forceinline__ uint32_t e4m3fn_to_bf16_bits(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 8;
  const uint32_t e = (b >> 3) & 0xFu;
  const uint32_t m = b & 0x7u;
  if ((b & 0x7Fu) == 0x7Fu) return sign | 0x7FC0u;     // NaN
  if (e != 0) return sign | ((e + 120u) << 7) | (m << 4);
  if (m == 0) return sign;                               // +-0
  // subnormal m * 2^-9: normalise on the leading bit p of m
  const uint32_t p = 31u - __builtin_clz(m);
  return sign | ((118u + p) << 7) | ((m - (1u << p)) << (7u - p));
}

// 8 E4M3FN bytes (two dwords) -> 8 BF16 values packed in four dwords.
__device__ __forceinline__ u32x4 widen_e4m3fn_x8(u32x2 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i >> 1] >> ((i & 1) * 16);
    r[i] = e4m3fn_to_bf16_bits(w & 0xFFu) |
           (e4m3fn_to_bf16_bits((w >> 8) & 0xFFu) << 16);
  }
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;   // round to nearest even
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);    // v_log_f32 (base 2)
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

// Byte offset of element 0 of 16-B chunk `chunk` (0..63) of tile row `row`.
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * kRowPitch + (chunk << 4);
}

// Row of k-slot (g, j) of a 32-row tile in the PV operands: slot j < 4 is
// row 4g+j of the first 16-row block, j >= 4 row 4g+j-4 of the second, the
// order in which the S^T accumulators hold them.
__device__ __forceinline__ int pv_row(int g, int j) {
  return (j < 4) ? (g * 4 + j) : (16 + g * 4 + (j - 4));
}

__device__ __forceinline__ void record_error(int32_t* err, int code, int t,
                                             int c) {
  if (atomicCAS(err, 0, code) == 0) {
    atomicExch(err + 1, t);
    atomicExch(err + 2, c);
  }
}

// ---------------------------------------------------------------------------
// split kernel
// ---------------------------------------------------------------------------

template <int HB, bool Q_FP8, bool KV_FP8, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1)
void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][kTileBytes];
  __shared__ int32_t slots[kSeg];
  __shared__ int32_t wave_cnt[4];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;       // 16-lane group: k-group of MFMA operands
  const int li = lane & 15;      // row / column inside a 16x16 block
  constexpr int H = 64 * HB;

  // XCD-aware mapping: the hardware hands consecutive workgroup ids to the
  // 8 XCDs round-robin, so give each XCD a contiguous range of work items;
  // the splits of one token and neighbouring tokens (which share rows in
  // speculative decode) then run together on one XCD and share its L2.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int q8 = nblk >> 3, r8 = nblk & 7;
  const int item = xcd * q8 + min(xcd, r8) + (blockIdx.x >> 3);
  const int t = item / p.S;
  const int s = item - t * p.S;

  const int head0 = wave * 16 * HB;

  int len = p.topk_lens ? p.topk_lens[t] : p.K;
  if (p.validate && threadIdx.x == 0 && s == 0 && (len < 0 || len > p.K))
    record_error(p.err, 2, t, -1);
  len = min(max(len, 0), p.K);
  const int c_begin = s * p.split_cols;
  const int c_end = min(len, c_begin + p.split_cols);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds head li and
  // dims [kk*32 + 8g, +8) for every 32-dim step kk.
  bf16x8 qf[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = head0 + hb * 16 + li;
    const size_t qrow = ((size_t)t * H + head) * kD;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int d0 = kk * 32 + g * 8;
      u32x4 v;
      if constexpr (Q_FP8) {
        const u32x2 raw = *(const u32x2*)((const uint8_t*)p.q + qrow + d0);
        v = widen_e4m3fn_x8(raw);
      } else {
        v = *(const u32x4*)((const uint16_t*)p.q + qrow + d0);
      }
      qf[hb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run[HB], l_run[HB];
  f32x4 o[32][HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m_run[hb] = -INFINITY;
    l_run[hb] = 0.f;
#pragma unroll
    for (int db = 0; db < 32; ++db) o[db][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int seg0 = c_begin; seg0 < c_end; seg0 += kSeg) {
    const int seg1 = min(c_end, seg0 + kSeg);

    // ---- compact the active slots of this segment into LDS ----------------
    __syncthreads();   // the previous segment's tiles no longer read slots[]
    int n_act = 0;
    for (int c0 = seg0; c0 < seg1; c0 += kThreads) {
      const int c = c0 + threadIdx.x;
      bool act = false;
      int code = 0;
      if (c < seg1) {
        const int r = p.indices[(int64_t)t * p.index_row_stride + c];
        if (r != -1) {
          const bool swa = c < kSwaColumns;
          const int64_t rows = swa ? p.swa_rows : p.comp_rows;
          if (r >= 0 && (int64_t)r < rows) {
            act = true;
            code = swa ? r : (int)((uint32_t)r | 0x80000000u);
          } else if (p.validate) {
            record_error(p.err, 1, t, c);
          }
        }
      }
      const uint64_t bal = __ballot(act);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[wave] = __popcll(bal);
      __syncthreads();
      int off = n_act, tot = 0;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const int cw = wave_cnt[w2];
        off += (w2 < wave) ? cw : 0;
        tot += cw;
      }
      if (act) slots[off + pre] = code;
      n_act += tot;
      __syncthreads();
    }

    // ---- gather + attend, 32 rows per tile ---------------------------------
    const int ntiles = (n_act + kTile - 1) / kTile;
    // Each wave stages 8 rows of a tile; lane `lane` carries 16-B chunk
    // `lane` of a BF16 row (8 bytes of an FP8 row, widened before LDS).
    u32x4 st16[8];
    u32x2 st8[8];

    auto load_tile = [&](int tile) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int si = tile * kTile + wave * 8 + jj;
        if (si < n_act) {
          const int code = slots[si];
          const uint8_t* base = code < 0 ? p.comp : p.swa;
          const int64_t row = (int64_t)(code & 0x7FFFFFFF);
          const uint8_t* src = base + row * p.row_stride_bytes;
          if constexpr (KV_FP8) st8[jj] = *(const u32x2*)(src + lane * 8);
          else st16[jj] = *(const u32x4*)(src + lane * 16);
        } else {
          if constexpr (KV_FP8) st8[jj] = u32x2{0u, 0u};
          else st16[jj] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = wave * 8 + jj;
        u32x4 v;
        if constexpr (KV_FP8) v = widen_e4m3fn_x8(st8[jj]);
        else v = st16[jj];
        *(u32x4*)(&kv_lds[buf][tile_off(j, lane)]) = v;
      }
    };

    if (ntiles > 0) {
      load_tile(0);
      store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      if (it + 1 < ntiles) load_tile(it + 1);    // in flight during compute
      const uint8_t* tb = kv_lds[buf];
      const int n_tile = min(kTile, n_act - it * kTile);

      // S^T[row, head] for 2 row blocks x HB head blocks
      f32x4 sacc[2][HB];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[rb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const bf16x8 a = *(const bf16x8*)(tb + tile_off(rb * 16 + li, kk * 4 + g));
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            sacc[rb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, qf[hb][kk], sacc[rb][hb], 0, 0, 0);
        }
      }

      // online softmax (base 2) per head; lane holds head li, rows 4g+i of
      // each row block
      bf16x8 pf[HB];
      float alpha[HB];
      bool need_any = false;
      float x[HB][8];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = rb * 16 + g * 4 + i;
            const float v = (row < n_tile) ? sacc[rb][hb][i] * p.scale_log2
                                           : -INFINITY;
            x[hb][rb * 4 + i] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool need = tmax > m_run[hb] + kRescaleThreshold;
        alpha[hb] = 1.f;
        if (need) {
          alpha[hb] = fast_exp2(m_run[hb] - tmax);
          m_run[hb] = tmax;
        }
        need_any |= need;
      }
      if (__ballot(need_any) != 0ull) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          l_run[hb] *= alpha[hb];
#pragma unroll
          for (int db = 0; db < 32; ++db) o[db][hb] *= alpha[hb];
        }
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float pv[8];
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp2(x[hb][j] - m_run[hb]);
          lsum += pv[j];
        }
        l_run[hb] += lsum;
        u32x4 packed;
#pragma unroll
        for (int k = 0; k < 4; ++k) packed[k] = pack_bf16x2(pv[2 * k], pv[2 * k + 1]);
        pf[hb] = __builtin_bit_cast(bf16x8, packed);
      }

      // O^T[d, head] += V^T[d, rows] * P^T[rows, head]
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const int d = db * 16 + li;
        const int chunk = d >> 3;
        const int sub = (d & 7) * 2;
        bf16x8 a;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = pv_row(g, j);
          a[j] = *(const __bf16*)(tb + tile_off(row, chunk) + sub);
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[hb], o[db][hb],
                                                              0, 0, 0);
      }

      if (it + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue ------------------------------------------------------------
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float l = l_run[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float m = m_run[hb];
    const int head = head0 + hb * 16 + li;
    float inv, lse;
    if constexpr (SPLIT) {
      inv = (l > 0.f) ? p.bmm2 / l : 0.f;
      lse = (l > 0.f) ? m + fast_log2(l) : -INFINITY;
    } else {
      float fac = 1.f;
      if (p.sinks) {
        const float sl = p.sinks[head] * kLog2e;
        const float mm = fmaxf(m, sl);
        fac = fast_exp2(m - mm);     // 0 when nothing was active (m = -inf)
        l = l * fac + fast_exp2(sl - mm);
        m = mm;
      }
      inv = (l > 0.f) ? fac * p.bmm2 / l : 0.f;
      lse = (l > 0.f) ? p.lse_scale * (m + fast_log2(l)) : -INFINITY;
    }
    uint16_t* dst;
    if constexpr (SPLIT)
      dst = p.mid_out + (((size_t)t * H + head) * p.S + s) * kD;
    else
      dst = (uint16_t*)p.out + ((size_t)t * H + head) * kD;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const f32x4 v = o[db][hb];
      u32x2 w;
      w[0] = pack_bf16x2(v[0] * inv, v[1] * inv);
      w[1] = pack_bf16x2(v[2] * inv, v[3] * inv);
      *(u32x2*)(dst + db * 16 + g * 4) = w;
    }
    if (g == 0) {
      if constexpr (SPLIT) p.mid_lse[((size_t)t * H + head) * p.S + s] = lse;
      else if (p.out_lse) p.out_lse[(size_t)t * H + head] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// combine kernel: one wave per (token, head); lane owns 8 output dims
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256)
void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.T * p.H) return;
  const int h = item % p.H;
  const float* ml = p.mid_lse + (size_t)item * p.stride;
  const float mine = (lane < p.S) ? ml[lane] : -INFINITY;
  float L = wave_max(mine);
  const float sl = p.sinks ? p.sinks[h] * kLog2e : -INFINITY;
  L = fmaxf(L, sl);
  float w = 0.f;
  if (lane < p.S && mine != -INFINITY) w = fast_exp2(mine - L);
  float W = wave_sum(w);
  if (p.sinks) W += fast_exp2(sl - L);

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const uint16_t* base = p.mid_out + (size_t)item * p.stride * kD + lane * 8;
  for (int s = 0; s < p.S; ++s) {
    const float ws = __shfl(w, s);
    if (ws == 0.f) continue;   // uniform across the wave
    const u32x4 v = *(const u32x4*)(base + (size_t)s * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += ws * __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += ws * __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  const float inv = (W > 0.f) ? 1.f / W : 0.f;
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *(u32x4*)(p.out + (size_t)item * kD + lane * 8) = r;
  if (lane == 0 && p.out_lse)
    p.out_lse[item] = (W > 0.f) ? p.lse_scale * (L + fast_log2(W)) : -INFINITY;
}

__global__ void clear_error_kernel(int32_t* err) {
  if (threadIdx.x < 4) err[threadIdx.x] = (threadIdx.x == 0) ? 0 : -1;
}

template <int HB, bool QF, bool KF>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.T * p.S));
  if (p.S > 1)
    hipLaunchKernelGGL((decode_kernel<HB, QF, KF, true>), grid, dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<HB, QF, KF, false>), grid, dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int q_dtype, int kv_dtype,
                         hipStream_t stream) {
  const bool qf = q_dtype != 0, kf = kv_dtype != 0;
  if (p.H == 64) {
    if (!qf && !kf) return launch_decode_t<1, false, false>(p, stream);
    if (qf && kf) return launch_decode_t<1, true, true>(p, stream);
    return launch_decode_t<1, false, true>(p, stream);
  }
  if (!qf && !kf) return launch_decode_t<2, false, false>(p, stream);
  if (qf && kf) return launch_decode_t<2, true, true>(p, stream);
  return launch_decode_t<2, false, true>(p, stream);
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

}  // namespace smla
