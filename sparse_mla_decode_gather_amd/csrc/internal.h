// Internal interface between the C-ABI layer (api.cpp) and the gfx950
// kernels (kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kHeadDim = 512;
constexpr int kSwaColumns = 128;
constexpr int kMaxSplits = 64;
constexpr int kErrBlockBytes = 256;
// kv dtype code of the 584-byte packed block-scaled FP8 rows
// (SMLA_DTYPE_PACKED_FP8_584)
constexpr int kKvPacked584 = 2;
// Scratch of the allocation-free decode, per GPU (SMLA_NOALLOC_SCRATCH_BYTES)
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

// Everything the split kernel needs, resolved on the host.
struct DecodeParams {
  const void* q;                 // [T, H, 512]
  const uint8_t* swa;            // pool base pointers (bytes)
  const uint8_t* comp;
  int64_t swa_rows;
  int64_t comp_rows;
  int64_t row_stride_bytes;      // bytes between consecutive pool rows
  const int32_t* indices;
  int64_t index_row_stride;      // elements
  const int32_t* topk_lens;      // may be null
  const float* sinks;            // may be null
  float scale_log2;              // bmm1_scale * log2(e)
  float bmm2;
  float lse_scale;
  void* out;                     // bf16 [T, H, 512]      (S == 1)
  float* out_lse;                // [T, H] or null        (S == 1)
  uint16_t* mid_out;             // bf16 [T, H, S, 512]   (S > 1)
  float* mid_lse;                // [T, H, S]             (S > 1)
  int32_t* err;                  // error block or null
  int32_t T, H, K, S;
  int32_t split_cols;            // columns per split
  int32_t validate;
  // The token's columns [0, K) split in two tables: columns < swa_cols read
  // `indices` (SWA pool), the others read `indices2` at column - swa_cols
  // (compressed pool).  segmented = 0, combined form: indices2 = indices +
  // 128 and topk_lens counts both.  1, two segments: topk_lens counts the
  // first table's active columns and lens2 the second's.  2, page table:
  // indices2 holds compressed-pool page IDs of page_size rows, topk_lens
  // counts the visible window and lens2 window + compressed slots.
  const int32_t* indices2;
  int64_t index_row_stride2;
  const int32_t* lens2;          // [T] or null
  int32_t swa_cols;
  int32_t K2;                    // columns of the second table (slots when paged)
  int32_t segmented;
  int32_t page_size;             // > 0 only when segmented == 2
  // H=128 kernel: start the items of an XCD longest first (set when the
  // grid has more items than the device has compute units)
  int32_t rank_items;
  // launch the serialized tile pipeline (SMLA_FLAG_SERIAL_PIPELINE: an
  // LDS-race check, combined table only); read by the host dispatch
  int32_t serial;
  // head tiles: 0, or 1 when each token runs as two 64-head halves (the
  // H=64 kernel on 2T virtual tokens: virtual token v is token v >> 1,
  // heads 64 (v & 1) ..; q, out and the partials keep their [T, 128, ...]
  // layout, which is [2T, 64, ...])
  int32_t head_shift;
};

struct CombineParams {
  const uint16_t* mid_out;       // bf16 [T, H, stride, 512]
  const float* mid_lse;          // [T, H, stride]
  const float* sinks;            // [H] or null
  float lse_scale;
  uint16_t* out;                 // bf16 [T, H, 512]
  float* out_lse;                // [T, H] or null
  int32_t T, H, S, stride;
};

// The combined-table builder, resolved on the host.
struct BuildParams {
  const int32_t* swa;            // [T, swa_stride] or null (W == 0)
  int64_t swa_stride;
  const int32_t* comp;           // [T, comp_stride] or null (K2 == 0)
  int64_t comp_stride;
  const int32_t* comp_lens;      // [T] or null
  const int32_t* block_tables;   // [num_requests, bt_stride] (local only)
  int64_t bt_stride;
  const int32_t* token_to_req;   // [T] or null
  const int32_t* valid;          // [T] or null
  int32_t* out;                  // [T, out_stride]
  int64_t out_stride;
  int32_t* out_lens;             // [T]
  int32_t* err;                  // error block or null
  int32_t T, W, K2;
  int32_t local;
  int32_t max_blocks, page_size, num_requests;
};

hipError_t launch_decode(const DecodeParams& p, int q_dtype, int kv_dtype,
                         hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
// The H=128 BF16 gather without arithmetic or output (measurement aid).
hipError_t launch_gather_only(const DecodeParams& p, hipStream_t stream);
hipError_t launch_clear_error(int32_t* err, hipStream_t stream);
hipError_t launch_build_indices(const BuildParams& p, hipStream_t stream);
// Device address of the allocation-free decode's scratch on the current
// device (kNoAllocScratchBytes, 256-B aligned); looked up once per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace smla
