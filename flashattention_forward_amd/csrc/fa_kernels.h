// Kernel parameter blocks and host-side launch wrappers of the gfx950 kernels.
// Shared by the kernel sources and the C-ABI front end (api.cpp). Host-only
// declarations: the front end also builds with a plain C++ compiler (the
// sanitizer build of the host logic), so only the runtime API header is used.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

enum class InType { bf16 = 0, f16 = 1 };
enum class OutType { bf16 = 0, f16 = 1, f32 = 2 };

// Prefill: q, o [B, Sq, Hq, D]; k, v [B, Skv, Hkv, D].
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;       // [B, Hq, Sq] or null
  void* part_o;     // [S, B, Sq, Hq, D] in the output type when n_splits > 1
  float* part_lse;  // [S, B, Sq, Hq]
  int B, Hq, Hkv, Sq, Skv;
  int waves;     // waves per workgroup: 4 or 8 (8 only for head size 128)
  int pack;      // query heads per workgroup (1, 2, 4 or 8; divides Hq / Hkv and waves)
  int pingpong;  // 8 waves: the two-group ping-pong schedule (prefill_pp.hip)
  int n_qtiles;  // ceil(Sq / (32 * waves / pack))
  int n_splits;  // key splits per query tile
  int q_neg;     // 1: the scale was negative; the kernel uses -Q and |scale|
  float scale;       // |scale|, multiplies q.k
  float scale_log2;  // |scale| * log2(e)
  // Explicit additive mask (input type) or null: element (b, i, j) at
  // mask[b * mask_bstride + i * mask_stride + j]; mask_stride and mask_bstride
  // are multiples of 8 and rows hold at least Skv rounded up to 8 elements.
  const void* mask;
  int64_t mask_bstride, mask_stride;
};

// Paged decode, separate K/V pool [P, 2, Hkv, page, D] (D = 128).
struct DecodeSplitParams {
  const void* q;  // [B, Sq, Hq, D]
  const void* pool;
  const int32_t* page_table;  // [B, max_pages]
  const int32_t* seq_lens;    // [B]
  void* o;                    // [B, Sq, Hq, D]
  float* lse;                 // [B, Hq, Sq] or null
  void* part_o;               // [S, B, Sq, Hq, D] in the 16-bit input type
  float* part_lse;            // [S, B, Sq, Hq]
  int B, Sq, Hq, Hkv, page_size, max_pages, num_pages, max_seq_len;
  int n_hblk;    // ceil(Sq * (Hq / Hkv) / 16) row blocks per K/V head
  int chunk;     // tokens per split (multiple of 32)
  int n_splits;
  int n_units;   // B * Hkv * n_hblk * n_splits
  int q_neg;
  float scale, scale_log2;
};

// Paged MLA decode, shared pool [P, page, 576]; K = row, V = row[0:512].
struct DecodeMlaParams {
  const void* q;  // [B, Sq, Hq, 576]
  const void* pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* o;  // [B, Hq, 512]
  float* lse;
  void* part_o;     // [S, B, Sq, Hq, 512] in the input's 16-bit type when n_splits > 1
  float* part_lse;  // [S, B, Sq, Hq]
  int B, Sq, Hq, page_size, max_pages, num_pages, max_seq_len;
  int heads_per_wg;  // query rows (new token x head) per workgroup: 64 or 32
  int n_hblk;        // ceil(Hq * Sq / heads_per_wg)
  int chunk;         // tokens per split (multiple of 32; <= MLA_MAX_CHUNK with 64 heads)
  int n_splits;
  int q_neg;
  float scale, scale_log2;
};

// Split-KV log-sum-exp combine. Rows are in output order r = (b * Sq + i) * Hq + h;
// part_o [S, rows, D], part_lse [S, rows]; o [rows, D]; lse index (b * Hq + h) * Sq + i.
struct CombineParams {
  const void* part_o;  // fp32, or the output's 16-bit type when part16
  int part16;
  const float* part_lse;
  void* o;
  float* lse;
  int rows, D, n_splits, Sq, Hq;
};

hipError_t launch_prefill(const PrefillParams& p, int D, InType it, OutType ot, bool causal,
                          hipStream_t stream);
// Per (head size, input type) prefill launchers, each compiled in its own file.
hipError_t launch_prefill_128_bf16(const PrefillParams& p, OutType ot, bool causal,
                                   hipStream_t stream);
hipError_t launch_prefill_128_f16(const PrefillParams& p, OutType ot, bool causal,
                                  hipStream_t stream);
hipError_t launch_prefill_64_bf16(const PrefillParams& p, OutType ot, bool causal,
                                  hipStream_t stream);
hipError_t launch_prefill_64_f16(const PrefillParams& p, OutType ot, bool causal,
                                 hipStream_t stream);
hipError_t launch_decode_split(const DecodeSplitParams& p, InType it, hipStream_t stream);
hipError_t launch_prefill_pp(const PrefillParams& p, InType it, OutType ot, bool causal,
                             hipStream_t stream);
hipError_t launch_decode_mla(const DecodeMlaParams& p, InType it, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, OutType ot, hipStream_t stream);

// Device address (for the current device) of the library's static split-KV
// scratch of NOALLOC_SCRATCH_BYTES, looked up once per device; allocates nothing.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;  // FA_DECODE_NOALLOC_SCRATCH_BYTES
hipError_t device_scratch(void** ptr);

// Tile constants the host planner needs.
// Prefill: each wave owns 32 query rows; a workgroup has 4 or 8 waves (128 or
// 256 query rows). With 8 waves (head size 128, one workgroup per CU) every
// K/V tile copied into LDS serves 256 query rows, which halves the L2-to-CU
// traffic per flop; 4 waves keep more workgroups for small problems.
constexpr int PF_BM_MIN = 128;
constexpr int PF_BN = 64;   // keys per prefill tile
constexpr int MLA_MAX_CHUNK = 2048;  // tokens per MLA split with 64 heads per workgroup
constexpr int DEC_TILE = 32;  // tokens per decode tile

}  // namespace fa
