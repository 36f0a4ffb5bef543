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

// A 16-token block: absolute positions [t0, t0 + 16), of which [lo, hi) count.
struct Block {
  int32_t t0, lo, hi;
};

// Operand registers of one block.
struct Tile {
  uint4 k[4];     // K rows: this lane's 64 bytes of token (lane & 15)
  uint2 v[8];     // V^T: channel 16c + (lane & 15), tokens 4*(lane>>4) .. +3
};

struct Ctx {
  PoolArgs pl;
  int32_t b, h;
  const int32_t* pt_row;
  int32_t max_pp;
};

// Loads the tile of block `blk`; returns false when its physical page is
// not valid (the block then contributes nothing).
__device__ __forceinline__ bool load_tile(const Ctx& c, const Block& blk, Tile& t) {
  const int32_t j = blk.t0 / c.pl.p;
  const int32_t slot_in_page = blk.t0 % c.pl.p;
  if (j < 0 || j / c.pl.r >= c.max_pp) return false;
  const int32_t phys = c.pt_row[j / c.pl.r];
  if (phys < 0 || phys >= c.pl.N) return false;
  const int32_t lp = j % c.pl.r;
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t head = (int64_t)phys * c.pl.hkv + c.h;
  const uint16_t* kp = c.pl.k + ((head * c.pl.P + lp * c.pl.p + slot_in_page + row) * kHeadDim + 32 * quad);
  const uint4* k4 = reinterpret_cast<const uint4*>(kp);
#pragma unroll
  for (int i = 0; i < 4; ++i) t.k[i] = k4[i];
  const uint16_t* vp = c.pl.v + ((head * c.pl.r + lp) * kHeadDim + row) * c.pl.p + slot_in_page + 4 * quad;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch)
    t.v[ch] = *reinterpret_cast<const uint2*>(vp + (int64_t)16 * ch * c.pl.p);
  return true;
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
  if (bm == -INFINITY) return;                    // no valid token (same for every lane)
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
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    uint2 w = t.v[ch];
    if (!full) {                                   // stale pool bytes must not reach the MFMA
      w.x &= (valid[0] ? 0x0000FFFFu : 0u) | (valid[1] ? 0xFFFF0000u : 0u);
      w.y &= (valid[2] ? 0x0000FFFFu : 0u) | (valid[3] ? 0xFFFF0000u : 0u);
    }
    s16x4 a;
    __builtin_memcpy(&a, &w, 8);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, st.o[ch], 0, 0, 0);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, st.o[ch], 0, 0, 0);
  }
}

// Number of 16-token blocks of the streaming set and the block at index v.
struct StreamSet {
  int32_t s0, w0, nb_sink, first_w, total;
  __device__ StreamSet(int32_t L, int32_t sink, int32_t window) {
    s0 = min(sink, L);
    w0 = max(sink, L - window);
    nb_sink = (s0 + kBlockTokens - 1) / kBlockTokens;
    first_w = w0 / kBlockTokens;
    const int32_t nb_win = L > w0 ? (L - 1) / kBlockTokens - first_w + 1 : 0;
    total = nb_sink + nb_win;
  }
  __device__ Block at(int32_t v, int32_t L) const {
    Block b;
    if (v < nb_sink) {
      b.t0 = v * kBlockTokens;
      b.lo = b.t0;
      b.hi = min(b.t0 + kBlockTokens, s0);
    } else {
      b.t0 = (first_w + v - nb_sink) * kBlockTokens;
      b.lo = max(b.t0, w0);
      b.hi = min(b.t0 + kBlockTokens, L);
    }
    return b;
  }
};

__device__ bool page_selected(const int32_t* sel, int32_t cnt, int32_t j) {
  int32_t lo = 0, hi = cnt;                        // ascending ids
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    const int32_t x = sel[mid];
    if (x == j) return true;
    if (x < j) lo = mid + 1; else hi = mid;
  }
  return false;
}

template <int BPI>
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

  Ctx c{pl, b, h, bt.pt + (int64_t)b * bt.max_pp, bt.max_pp};

  // query operand: Q[g][32*quad + 8*i .. +8], zero for g >= G
  bf16x8 qb[4];
  const int32_t hq = pl.hkv * G;
  if (g < G) {
    const uint4* q4 = reinterpret_cast<const uint4*>(q + ((int64_t)b * hq + h * G + g) * kHeadDim + 32 * quad);
#pragma unroll
    for (int i = 0; i < 4; ++i) { uint4 w = q4[i]; __builtin_memcpy(&qb[i], &w, 16); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { uint4 w = {0, 0, 0, 0}; __builtin_memcpy(&qb[i], &w, 16); }
  }

  State st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) st.o[ch] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool dynamic = plan.kind[h] != 0;
  const int32_t* sel = sel_pages + ((int64_t)b * pl.hkv + h) * plan.k_max;
  if (dynamic && it == plan.items_dyn - 1) {
    // tail item: tokens appended since the selection, outside selected pages
    const int32_t cnt = min(max(sel_count[(int64_t)b * pl.hkv + h], 0), plan.k_max);
    const int32_t ls = max(sel_len[b], 0);
    for (int32_t t0 = (ls / kBlockTokens) * kBlockTokens; t0 < L; t0 += kBlockTokens) {
      if (page_selected(sel, cnt, t0 / pl.p)) continue;
      Block blk{t0, max(t0, ls), min(t0 + kBlockTokens, L)};
      Tile t;
      if (load_tile(c, blk, t)) process_tile(blk, t, qb, st);
    }
  } else if (L > 0) {
    int32_t total, v0 = it * BPI;
    StreamSet ss(L, plan.sink, plan.window);
    const int32_t sb = pl.p / kBlockTokens;
    const int32_t n_pages = (L + pl.p - 1) / pl.p;
    int32_t cnt = 0;
    if (dynamic) {
      cnt = min(max(sel_count[(int64_t)b * pl.hkv + h], 0), plan.k_max);
      total = cnt * sb;
    } else {
      total = ss.total;
    }
    const int32_t v1 = min(total, v0 + BPI);
    auto block_at = [&](int32_t v) -> Block {
      if (!dynamic) return ss.at(v, L);
      const int32_t j = sel[v / sb];
      Block blk{0, 0, 0};
      if (j < 0 || j >= n_pages) return blk;          // out of range: empty block
      blk.t0 = j * pl.p + (v % sb) * kBlockTokens;
      blk.lo = blk.t0;
      blk.hi = min(blk.t0 + kBlockTokens, L);
      return blk;
    };
    if (v0 < v1) {
      Block cur = block_at(v0);
      Tile tc;
      bool okc = cur.lo < cur.hi && load_tile(c, cur, tc);
      for (int32_t v = v0; v < v1; ++v) {
        Block nxt;
        Tile tn;
        bool okn = false;
        if (v + 1 < v1) {
          nxt = block_at(v + 1);
          okn = nxt.lo < nxt.hi && load_tile(c, nxt, tn);
        }
        if (okc) process_tile(cur, tc, qb, st);
        cur = nxt;
        tc = tn;
        okc = okn;
      }
    }
  }

  // fold the four token quads of the running sum
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  if (g < G) {
    const int64_t slot = (((int64_t)b * pl.hkv + h) * plan.item_stride + it) * G + g;
    float* o = part_o + slot * kHeadDim + 4 * quad;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) *reinterpret_cast<f32x4*>(o + 16 * ch) = st.o[ch];
    if (quad == 0) {
      part_ml[slot * 2 + 0] = st.m;
      part_ml[slot * 2 + 1] = st.l;
    }
  }
}

// Merge of the item partials of one query head: thread d owns channel d.
__global__ void __launch_bounds__(128) combine_kernel(int32_t hkv, AttnPlan plan, int32_t G,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse) {
  const int32_t hq = hkv * G;
  const int32_t b = blockIdx.x / hq, i = blockIdx.x % hq;
  const int32_t h = i / G, g = i % G;
  const int32_t n_items = plan.kind[h] ? plan.items_dyn : plan.items_stream;
  const int64_t slot0 = ((int64_t)b * hkv + h) * plan.item_stride;
  float M = -INFINITY;
  for (int32_t it = 0; it < n_items; ++it) M = fmaxf(M, part_ml[((slot0 + it) * G + g) * 2]);
  const int d = threadIdx.x;
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int32_t it = 0; it < n_items; ++it) {
      const int64_t slot = (slot0 + it) * G + g;
      const float w = __builtin_amdgcn_exp2f(part_ml[slot * 2] - M);
      den += w * part_ml[slot * 2 + 1];
      num += w * part_o[slot * kHeadDim + d];
    }
  }
  const int64_t oi = (int64_t)b * hq + i;
  out[oi * kHeadDim + d] = M == -INFINITY ? 0.f : num / den;
  if (lse && d == 0) lse[oi] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * kLn2;
}

template <int BPI>
hipError_t launch_attn_bpi(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan,
                           int32_t G, const uint16_t* q, const int32_t* sel_pages,
                           const int32_t* sel_count, const int32_t* sel_len, float* part_o,
                           float* part_ml, hipStream_t s) {
  const int64_t grid = (int64_t)batch.B * plan.items_per_seq;
  hipLaunchKernelGGL(attn_kernel<BPI>, dim3((unsigned)grid), dim3(64), 0, s, pool, batch, plan, G, q,
                     sel_pages, sel_count, sel_len, part_o, part_ml);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                       const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                       const int32_t* sel_len, float* out, float* lse, float* part_o,
                       float* part_ml, hipStream_t s) {
  if (batch.B == 0) return hipSuccess;
  hipError_t e;
  switch (plan.blocks_per_item) {
    case 4: e = launch_attn_bpi<4>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, s); break;
    case 8: e = launch_attn_bpi<8>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, s); break;
    case 16: e = launch_attn_bpi<16>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(batch.B * pool.hkv * G), dim3(128), 0, s, pool.hkv, plan, G,
                     part_o, part_ml, out, lse);
  return hipGetLastError();
}

}  // namespace spa
