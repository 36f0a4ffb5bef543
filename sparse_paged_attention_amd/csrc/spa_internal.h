// Internal declarations shared by the host dispatch (api.cpp) and the kernel
// files. Not part of the public ABI (include/spa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spa.h"

namespace spa {

constexpr int kHeadDim = 128;       // D
constexpr int kBlockTokens = 16;    // tokens per attention block (MFMA M/K tile)
constexpr int kMaxKvHeads = 128;

// Pool geometry and base pointers, passed by value to every kernel.
struct PoolArgs {
  int32_t hkv;      // KV heads
  int32_t hs;       // head slots per physical page: hkv, or fewer when the page table's pages hold the
                    // dynamic heads and the streaming heads' rings the streaming heads (slot = rank in kind)
  int32_t p;        // logical page (tokens)
  int32_t P;        // physical page (tokens)
  int32_t r;        // P / p
  int32_t N;        // physical pages
  uint16_t* k;      // [N][hs][P][D]
  uint16_t* v;      // [N][hs][r][D][p]
  uint16_t* summ;   // [N][hs][r][2][D]
  int32_t q8;       // 1: k and v hold E4M3 codes (bytes, same layouts) with row scales ks / vs
  float* ks;        // [N][hs][P] key row scales (q8)
  float* vs;        // [N][hs][P] value row scales (q8)
};

struct BatchArgs {
  int32_t B;
  int32_t max_pp;
  const int32_t* pt;    // [B][max_pp]
  const int32_t* lens;  // [B]
  // Streaming heads kept in a ring of physical pages per sequence (NULL: in
  // the pages of the page table like dynamic heads): ring[b] is the first of
  // ring_sink + ring_win consecutive pages; position t of a streaming head is
  // in page ring[b] + (t/P < ring_sink ? t/P : ring_sink + (t/P - ring_sink) % ring_win).
  const int32_t* ring;
  int32_t ring_sink, ring_win;
};

// A list of KV-head ids (dynamic heads for selection / summaries).
struct HeadList {
  int32_t n;
  int16_t id[kMaxKvHeads];
};

// Work plan of the attention launch: every streaming head is cut into
// items_stream items and every dynamic head into items_dyn items (the last of
// which covers the tokens appended since the selection). Work-groups are
// numbered [sequence][KV head][item], each head holding as many items as its
// kind needs; partials are stored item_stride slots per head.
struct AttnPlan {
  int32_t items_stream;         // items per streaming head
  int32_t items_dyn;            // items per dynamic head
  int32_t item_stride;          // max(items_stream, items_dyn): partial slots per head
  int32_t items_per_seq;        // sum over the KV heads of their item counts
  int32_t blocks_per_item;      // 16-token blocks per item
  int32_t sink, window;
  int32_t k_max;
  uint32_t dyn_mask[kMaxKvHeads / 32];   // bit h set: KV head h is dynamic
  int32_t use_phys;                      // selected pages' physical pages come with the selection
  int32_t extra_partial;                 // 1: slot items_* of each head holds an appended token's partial
  int64_t sel_mask;                      // ~0 with dynamic heads, 0 without (selection unused)
};

// Prefill block-sparse attention (spa_prefill_attn): a sequence's queries
// [H_q][L][D] and keys / values [H_kv][L][D] in position order.
constexpr int kPrefillBlock = 64;              // tokens per query / key block
constexpr int kPrefillMaxBlocks = 8192;        // blocks a selection row holds (L <= 524288)

struct PrefillArgs {
  int32_t hq, hkv, G;
  int64_t L;
  int32_t nb;                 // blocks: ceil(L / 64)
  int32_t kb;                 // key blocks per query block, the diagonal one included
  int32_t sink, window;       // streaming heads
  int32_t dense;              // 1: dynamic heads attend every earlier token (no selection)
  int32_t any_dynamic;
  uint32_t dyn_mask[kMaxKvHeads / 32];
  const uint16_t* q;          // [H_q][L][D]
  const uint16_t* k;          // [H_kv][L][D]
  const uint16_t* v;
  const uint16_t* wq;         // [D][D / 8]
  const uint16_t* wk;
  double* qp;                 // [H_kv][nb][D / 8]: projected group-mean queries of each block
  double* kp;                 // [H_kv][nb][D / 8]: projected mean keys
  int32_t* sel;               // [H_kv][nb][kb]: attended key blocks of each query block, ascending
  int32_t* cnt;               // [H_kv][nb]
  float* scores;              // NULL or [H_kv][nb][nb]: block scores (entries i < j)
  float* out;                 // [H_q][L][D]
  float* lse;                 // NULL or [H_q][L]
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// Bytes of the static scratch array of the attention entry point that
// allocates nothing (spa_sparse_decode_attn_noalloc), per GPU.
constexpr size_t kScratchBytes = SPA_NOALLOC_SCRATCH_BYTES;

// Device address of that array on the current device (looked up once per
// device) and its size.
hipError_t scratch_area(void** ptr, size_t* bytes);

// ---- launchers (return hipError_t of the launch) -------------------------
hipError_t launch_append(const PoolArgs& pool, const BatchArgs& batch,
                         const uint16_t* k_new, const uint16_t* v_new,
                         const HeadList* dyn, hipStream_t s);
hipError_t launch_write(const PoolArgs& pool, const int32_t* pt_row, int64_t start,
                        int64_t count, const uint16_t* k, const uint16_t* v,
                        const HeadList* dyn,                  // NULL or dynamic heads: summaries too
                        int32_t ring_base, int32_t ring_sink,  // ring_base < 0: no ring
                        int32_t ring_win, hipStream_t s);
hipError_t launch_summary(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                          const int32_t* first_pos, int32_t max_tokens, hipStream_t s);
hipError_t launch_select(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                         int32_t G, const uint16_t* q, const int32_t* budget, int32_t k_max,
                         int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len,
                         int32_t* sel_phys, float* scores, int32_t n_max,
                         const uint16_t* k_new, const uint16_t* v_new,   // NULL: no token appended
                         hipStream_t s);
hipError_t launch_attn(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan,
                       int32_t G, const uint16_t* q, const int32_t* sel_pages,
                       const int32_t* sel_count, const int32_t* sel_len,
                       const int32_t* sel_phys, float* out,
                       float* lse, float* part_o, float* part_ml,
                       const uint16_t* k_new, const uint16_t* v_new,   // NULL: no token appended
                       hipStream_t s);

}  // namespace spa
