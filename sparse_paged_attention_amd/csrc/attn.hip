// Unified sparse decode attention over the paged pool.
//
// One launch serves both head kinds (LServe write-up, bqwf.cn, "2.1": a fused
// block-sparse kernel handles static and dynamic sparsity together):
//   streaming head: tokens [0, min(sink, L)) U [max(sink, L - window), L)
//   dynamic head:   tokens of the selected logical pages (positions < L), plus
//                   the tokens appended since the selection, [L_s, L).
// Work is cut into items of a few 16-token blocks; each item runs the online
// softmax over its blocks and writes a partial (running max, running sum,
// unnormalised output), and a second kernel merges the partials of each query
// head (FlashAttention's tiled online softmax, long-context survey
// xllm-io.github.io "2.1"; the row-max / row-sum outputs of the Novita vLLM
// article, "2. 注意力机制修改").
//
// Per 16-token block one wave issues
//   S^T[16 tok][16 q] = K[16][128] . Q^T      4 x v_mfma_f32_16x16x32_bf16
//   O^T[128][16 q]   += V^T[128][16] . P^T    8 x 2 x v_mfma_f32_16x16x16_bf16
// The query group (G <= 16 heads sharing the KV head, grouped-query attention
// of the long-context survey "2.3") fills the 16 query columns; P is split
// into bf16 high and low parts so the products keep ~16 significant bits.
// Keys are stored token-major and values channel-major per logical page, so
// both tiles load straight from HBM into operand registers.
#include "spa_internal.h"

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// log2(e) / sqrt(128): scores are kept in the log2 domain
constexpr float kScaleLog2 = 0.12751743074602467f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ int32_t clamp_len(const BatchArgs& bt, int32_t b, int32_t P) {
  int32_t L = bt.lens[b];
  int32_t cap = bt.max_pp * P;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A 16-token block: absolute positions [t0, t0 + 16), of which [lo, hi) count,
// in physical page `phys` (already validated) at logical slot `lp`.
struct Block {
  int32_t t0, lo, hi, phys, lp;
};

// Operand registers of one block.
struct Tile {
  uint4 k[4];     // K rows: this lane's 64 bytes of token (lane & 15)
  uint2 v[8];     // V^T: channel 16c + (lane & 15), tokens 4*(lane>>4) .. +3
};

// Issues the loads of a block's tile. Empty blocks load from page 0 of the
// pool (always mapped), so the loads never depend on control flow.
template <int PG>
__device__ __forceinline__ void issue_tile(const PoolArgs& pl, int32_t h, const Block& blk, Tile& t) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t head = (int64_t)blk.phys * pl.hkv + h;
  const int32_t in_page = blk.t0 & (PG - 1);
  const uint4* k4 = reinterpret_cast<const uint4*>(
      pl.k + ((head * pl.P + blk.lp * PG + in_page + row) * kHeadDim + 32 * quad));
#pragma unroll
  for (int i = 0; i < 4; ++i) t.k[i] = k4[i];
  const uint16_t* vp = pl.v + ((head * pl.r + blk.lp) * kHeadDim + row) * PG + in_page + 4 * quad;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) t.v[ch] = *reinterpret_cast<const uint2*>(vp + 16 * ch * PG);
}

struct State {
  float m;          // running max of this lane's query, log2 domain
  float l;          // running sum over this lane's tokens
  f32x4 o[8];       // O^T: channels 16c + 4*quad + r of query (lane & 15)
};

__device__ __forceinline__ void process_tile(const Block& blk, const Tile& t, const bf16x8 (&qb)[4],
                                             State& st) {
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 a;
    __builtin_memcpy(&a, &t.k[i], 16);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[i], s, 0, 0, 0);
  }
  // lane holds scores of tokens t0 + 4*quad + r for query (lane & 15)
  float x[4];
  bool valid[4];
  float bm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int32_t tok = blk.t0 + 4 * quad + r;
    valid[r] = tok >= blk.lo && tok < blk.hi;
    x[r] = valid[r] ? s[r] * kScaleLog2 : -INFINITY;
    bm = fmaxf(bm, x[r]);
  }
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  // a non-empty block has a valid token, so bm is finite
  const float m_new = fmaxf(st.m, bm);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float pr[4];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pr[r] = valid[r] ? __builtin_amdgcn_exp2f(x[r] - m_new) : 0.f;
    psum += pr[r];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) st.o[ch] *= alpha;

  s16x4 phi, plo;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint16_t hb = bf16_rne(pr[r]);
    const float rest = pr[r] - __uint_as_float((uint32_t)hb << 16);
    phi[r] = (short)hb;
    plo[r] = (short)bf16_rne(rest);
  }
  const bool full = blk.lo <= blk.t0 && blk.hi >= blk.t0 + kBlockTokens;
  const uint32_t mx = (valid[0] ? 0x0000FFFFu : 0u) | (valid[1] ? 0xFFFF0000u : 0u);
  const uint32_t my = (valid[2] ? 0x0000FFFFu : 0u) | (valid[3] ? 0xFFFF0000u : 0u);
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    uint2 w = t.v[ch];
    if (!full) {                                   // stale pool bytes must not reach the MFMA
      w.x &= mx;
      w.y &= my;
    }
    s16x4 a;
    __builtin_memcpy(&a, &w, 8);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, st.o[ch], 0, 0, 0);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, st.o[ch], 0, 0, 0);
  }
}

__device__ __forceinline__ bool page_selected(const int32_t* sel, int32_t cnt, int32_t j) {
  int32_t lo = 0, hi = cnt;                        // ascending ids
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    const int32_t x = sel[mid];
    if (x == j) return true;
    if (x < j) lo = mid + 1; else hi = mid;
  }
  return false;
}

// Which blocks an item covers. Blocks are numbered per head:
//   streaming: the sink blocks, then the window blocks;
//   dynamic:   block (i, s) = 16-token block s of the i-th selected page;
//   tail:      16-token blocks of [floor16(L_s), L) outside selected pages.
struct BlockSource {
  int32_t kind;          // 0 streaming, 1 dynamic, 2 tail
  int32_t L, PG;
  int32_t s0, w0, nb_sink, first_w;          // streaming
  const int32_t* sel;
  int32_t cnt;                               // dynamic / tail
  int32_t ls_floor, ls;                      // tail
  int32_t n_pages;

  // token range of block v (lo == hi: empty); t0 is 16-aligned
  __device__ __forceinline__ void range(int32_t v, int32_t& t0, int32_t& lo, int32_t& hi) const {
    if (kind == 0) {
      if (v < nb_sink) {
        t0 = v * kBlockTokens; lo = t0; hi = min(t0 + kBlockTokens, s0);
      } else {
        t0 = (first_w + v - nb_sink) * kBlockTokens; lo = max(t0, w0); hi = min(t0 + kBlockTokens, L);
      }
    } else if (kind == 1) {
      const int32_t sb = PG / kBlockTokens;
      const int32_t j = sel[v / sb];
      if (j < 0 || j >= n_pages) { t0 = 0; lo = 0; hi = 0; return; }
      t0 = j * PG + (v % sb) * kBlockTokens; lo = t0; hi = min(t0 + kBlockTokens, L);
    } else {
      t0 = ls_floor + v * kBlockTokens;
      lo = max(t0, ls); hi = min(t0 + kBlockTokens, L);
      if (page_selected(sel, cnt, t0 / PG)) hi = lo;
    }
  }
};

// Resolves blocks [v0, v0 + BPI) (those at or past v_end are empty) to pool
// locations, then runs them through a two-tile software pipeline: the loads
// of block u+1 are in flight while block u is computed.
template <int PG, int BPI>
__device__ __forceinline__ void run_blocks(const PoolArgs& pl, const int32_t* pt_row, int32_t max_pp,
                                           int32_t h, const BlockSource& src, int32_t v0, int32_t v_end,
                                           const bf16x8 (&qb)[4], State& st) {
  Block blk[BPI];
#pragma unroll
  for (int u = 0; u < BPI; ++u) {
    int32_t t0 = 0, lo = 0, hi = 0;
    if (v0 + u < v_end) src.range(v0 + u, t0, lo, hi);
    const int32_t j = t0 / PG;
    const int32_t slot = j / (pl.P / PG);
    int32_t phys = (lo < hi && slot < max_pp) ? pt_row[slot] : -1;
    if (phys < 0 || phys >= pl.N) { phys = 0; hi = lo; t0 = 0; }
    blk[u] = Block{t0, lo, hi, phys, j % (pl.P / PG)};
    if (hi <= lo) blk[u].lp = 0;
  }
  Tile ta, tb;
  issue_tile<PG>(pl, h, blk[0], ta);
#pragma unroll
  for (int u = 0; u < BPI; u += 2) {
    if (u + 1 < BPI) issue_tile<PG>(pl, h, blk[u + 1], tb);
    if (blk[u].lo < blk[u].hi) process_tile(blk[u], ta, qb, st);
    if (u + 2 < BPI) issue_tile<PG>(pl, h, blk[u + 2], ta);
    if (u + 1 < BPI && blk[u + 1].lo < blk[u + 1].hi) process_tile(blk[u + 1], tb, qb, st);
  }
}

// One item of one (sequence, KV head): the online softmax over its blocks and
// a partial (max, sum, unnormalised output) per query head.
template <int PG, int BPI>
__global__ void __launch_bounds__(64) attn_kernel(PoolArgs pl, BatchArgs bt, AttnPlan plan, int32_t G,
                                                  const uint16_t* __restrict__ q,
                                                  const int32_t* __restrict__ sel_pages,
                                                  const int32_t* __restrict__ sel_count,
                                                  const int32_t* __restrict__ sel_len,
                                                  float* __restrict__ part_o,
                                                  float* __restrict__ part_ml) {
  const int32_t b = blockIdx.x / plan.items_per_seq;
  const int32_t rem = blockIdx.x % plan.items_per_seq;
  int32_t h = 0;
  while (plan.item_base[h + 1] <= rem) ++h;
  const int32_t it = rem - plan.item_base[h];
  const int32_t L = clamp_len(bt, b, pl.P);
  const int lane = threadIdx.x & 63;
  const int g = lane & 15, quad = lane >> 4;
  const int32_t* pt_row = bt.pt + (int64_t)b * bt.max_pp;

  // query operand: Q[g][32*quad + 8*i .. +8], zero for g >= G
  bf16x8 qb[4];
  const int32_t hq = pl.hkv * G;
  {
    const int32_t gq = g < G ? g : 0;
    const uint4* q4 = reinterpret_cast<const uint4*>(q + ((int64_t)b * hq + h * G + gq) * kHeadDim + 32 * quad);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = q4[i];
      if (g >= G) w = uint4{0, 0, 0, 0};
      __builtin_memcpy(&qb[i], &w, 16);
    }
  }

  State st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) st.o[ch] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool dynamic = plan.kind[h] != 0;
  const int32_t n_items = dynamic ? plan.items_dyn : plan.items_stream;
  BlockSource src;
  src.L = L;
  src.PG = PG;
  src.n_pages = (L + PG - 1) / PG;
  src.sel = sel_pages + ((int64_t)b * pl.hkv + h) * plan.k_max;
  src.cnt = 0;
  if (L > 0) {
    if (!dynamic) {
      src.kind = 0;
      src.s0 = min(plan.sink, L);
      src.w0 = max(plan.sink, L - plan.window);
      src.nb_sink = (src.s0 + kBlockTokens - 1) / kBlockTokens;
      src.first_w = src.w0 / kBlockTokens;
      const int32_t nb_win = L > src.w0 ? (L - 1) / kBlockTokens - src.first_w + 1 : 0;
      run_blocks<PG, BPI>(pl, pt_row, bt.max_pp, h, src, it * BPI, src.nb_sink + nb_win, qb, st);
    } else {
      src.cnt = min(max(sel_count[(int64_t)b * pl.hkv + h], 0), plan.k_max);
      if (it < n_items - 1) {
        src.kind = 1;
        run_blocks<PG, BPI>(pl, pt_row, bt.max_pp, h, src, it * BPI, src.cnt * (PG / kBlockTokens), qb, st);
      } else {
        src.kind = 2;
        src.ls = min(max(sel_len[b], 0), L);
        src.ls_floor = (src.ls / kBlockTokens) * kBlockTokens;
        const int32_t nb = (L - src.ls_floor + kBlockTokens - 1) / kBlockTokens;
        for (int32_t v0 = 0; v0 < nb; v0 += BPI)
          run_blocks<PG, BPI>(pl, pt_row, bt.max_pp, h, src, v0, nb, qb, st);
      }
    }
  }

  // fold the four token quads of the running sum, store the partial
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  const int64_t slot0 = ((int64_t)b * pl.hkv + h) * plan.item_stride * G;
  if (g < G) {
    const int64_t slot = slot0 + (int64_t)it * G + g;
    float* o = part_o + slot * kHeadDim + 4 * quad;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) *reinterpret_cast<f32x4*>(o + 16 * ch) = st.o[ch];
    if (quad == 0) {
      part_ml[slot * 2 + 0] = st.m;
      part_ml[slot * 2 + 1] = st.l;
    }
  }

}

// Merge of the item partials of one (sequence, KV head): the running-max /
// running-sum rule of online softmax applied across items. Thread (g, d) owns
// channel d of query g; the items' (max, sum) pairs are staged in LDS first so
// every output channel's loads are independent and in flight together.
constexpr int kCombineThreads = 512;
constexpr int kMaxItemsLds = kMaxPartialsPerHead;

__global__ void __launch_bounds__(kCombineThreads) combine_kernel(int32_t hkv, AttnPlan plan, int32_t G,
                                                                  const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse) {
  __shared__ float sm[kMaxItemsLds], sl[kMaxItemsLds];
  __shared__ float sM[16];
  const int32_t b = blockIdx.x / hkv, h = blockIdx.x % hkv;
  const int32_t n_items = plan.kind[h] ? plan.items_dyn : plan.items_stream;
  const int64_t slot0 = ((int64_t)b * hkv + h) * plan.item_stride * G;   // slot(i, g) = slot0 + i*G + g
  const int32_t n_ml = n_items * G;                                     // <= kMaxItemsLds (host check)
  for (int32_t k = threadIdx.x; k < n_ml; k += kCombineThreads) {
    sm[k] = part_ml[(slot0 + k) * 2];
    sl[k] = part_ml[(slot0 + k) * 2 + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY;
    for (int32_t i = 0; i < n_items; ++i) M = fmaxf(M, sm[i * G + threadIdx.x]);
    sM[threadIdx.x] = M;
  }
  __syncthreads();
  const int32_t hq = hkv * G;
  for (int32_t gd = threadIdx.x; gd < G * kHeadDim; gd += kCombineThreads) {
    const int32_t g = gd / kHeadDim, d = gd % kHeadDim;
    const float M = sM[g];
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
      for (int32_t i = 0; i < n_items; ++i) {
        const float w = __builtin_amdgcn_exp2f(sm[i * G + g] - M);
        den += w * sl[i * G + g];
        num += w * part_o[(slot0 + (int64_t)i * G + g) * kHeadDim + d];
      }
    }
    const int64_t oi = (int64_t)b * hq + h * G + g;
    out[oi * kHeadDim + d] = M == -INFINITY ? 0.f : num / den;
    if (lse && d == 0) lse[oi] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * kLn2;
  }
}

template <int PG, int BPI>
hipError_t launch_attn_t(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                         const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                         const int32_t* sel_len, float* part_o, float* part_ml, int32_t* tickets,
                         float* out, float* lse, hipStream_t s) {
  const int64_t grid = (int64_t)batch.B * plan.items_per_seq;
  hipLaunchKernelGGL((attn_kernel<PG, BPI>), dim3((unsigned)grid), dim3(64), 0, s, pool, batch, plan, G, q,
                     sel_pages, sel_count, sel_len, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(batch.B * pool.hkv), dim3(kCombineThreads), 0, s, pool.hkv, plan, G,
                     part_o, part_ml, out, lse);
  return hipGetLastError();
}

template <int PG>
hipError_t launch_attn_p(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                         const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                         const int32_t* sel_len, float* part_o, float* part_ml, int32_t* tickets,
                         float* out, float* lse, hipStream_t s) {
  switch (plan.blocks_per_item) {
    case 4: return launch_attn_t<PG, 4>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 8: return launch_attn_t<PG, 8>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 16: return launch_attn_t<PG, 16>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                       const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                       const int32_t* sel_len, float* out, float* lse, float* part_o,
                       float* part_ml, int32_t* tickets, hipStream_t s) {
  if (batch.B == 0) return hipSuccess;
  switch (pool.p) {
    case 16: return launch_attn_p<16>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 32: return launch_attn_p<32>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 64: return launch_attn_p<64>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spa
