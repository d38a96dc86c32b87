// Device-side building blocks of the sparse decode attention (split and merge
// workgroups), shared by the attention kernels and the fused kernels of the
// overlapped step.  Internal to liboasis; the design notes are in attention.hip.
#pragma once

#include "common.h"
#include "launch.h"

namespace oasis {

constexpr int kAttnWaves = kWavesPerWG;                 // one 16-token unit per wave and round
constexpr int kAttnMaxSplits = 256;           // partials per head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short bf16x4_bits __attribute__((ext_vector_type(4)));

constexpr int kRec = kHeadDim + 4;  // workspace record: output (128), max, sum, padding

// Buffer resource over one head's K or V blocks; an offset at or past `bytes` reads
// zeros and touches no memory.
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOffMasked = 0x80000000u;
constexpr int kNtAux = 2;  // non-temporal: K and V are read once

// A wave's unit of work is 16 tokens of the table: one 16-token block, two 8-token
// blocks, or a 16-token chunk of a 32- or 64-token block.  It is taken as two
// halves of 8 tokens, each resolved on its own to a block and the 8-token
// sub-block inside it, so every block size runs the same code.
//
// K and V units are read with contiguous 1 KB wave loads (instruction s of a unit
// covers tokens 4s..4s+3, s < 2 in the first half): lane l holds token 4s + l/16,
// 16-byte chunk l%16.  That is already the layout the PV product wants for V.  For QK, lane l
// must supply one token's chunks, so K goes through LDS (rows padded to 272
// bytes, conflict-free) and is read back with MFMA row i holding token
// 4*(i%4) + i/4; the scores then come out with lane l owning exactly the tokens
// 4r + l/16 whose V rows it loaded.
constexpr int kKRow = kHeadDim * 2 / 16 + 1;  // padded LDS row of one K token, in 16-byte chunks

#ifndef OASIS_ATTN_MIN_WAVES
#define OASIS_ATTN_MIN_WAVES 4  // <= 128 VGPRs: four waves per SIMD
#endif
// GP: query heads per KV head rounded up to 4, 8 or 16 (sizes the LDS partials).
// RES: the entries are not a compacted table but the resident slots followed by the
// window blocks: entry e < K is slot e of `table` (rows of K, -1 = empty; a block at
// or past the first window block counts as a window block only), entry K + i is
// window block w0 + i.  `table_count` is unused then and T = K + the most window
// blocks a sequence can have.
template <int GP>
struct AttnShared {
  u32x4 kst[kAttnWaves][16 * kKRow];  // per-wave K staging (16 tokens)
  // Per-wave partials: the waves merge without a barrier; the last one to finish
  // combines them and writes the record, the others end as soon as they have
  // published theirs (freeing their slots for waves of other workgroups).
  alignas(16) float sm_o[kAttnWaves][GP][kHeadDim + 4];
  float sm_m[kAttnWaves][GP];
  float sm_l[kAttnWaves][GP];
  int arrived;
};

// Arguments of the attention split work.
struct AttnArgs {
  const u32x4* q;
  const char* k;
  const char* v;
  const int32_t* table;
  const int32_t* table_count;
  int T;
  const int32_t* seq_lens;
  float scale_log2;
  float* part;
  int heads, group, queries, NB, nsplit, rounds, K, window, bshift;
  // POOL only: the window ring (`k` and `v` are then the pool) and its slots per head.
  const char* ring_k;
  const char* ring_v;
  int WB;
};

// One workgroup of split `sp` of (sequence, KV head) `bh`; a wave that does not
// finish last returns early.  Every thread of the workgroup calls it.
// POOL (with RES): the blocks are read from the working set in HBM instead of the
// full cache: resident slot e from pool slot e (`k`, `v`: [B, H, K, bs, 128]),
// window block j from ring slot j % WB (`ring_k`, `ring_v`: [B, H, WB, bs, 128]).
template <int GP, bool RES, bool POOL = false>
__device__ __attribute__((always_inline)) void attn_split_wg(int sp, int bh, AttnShared<GP>& sh,
                                                             const AttnArgs& a) {
  static_assert(RES || !POOL, "the pool is addressed through the resident slots");
  const u32x4* __restrict__ q = a.q;
  const char* __restrict__ k = a.k;
  const char* __restrict__ v = a.v;
  const int32_t* __restrict__ table = a.table;
  const int T = a.T, heads = a.heads, group = a.group, queries = a.queries, NB = a.NB;
  const int nsplit = a.nsplit, rounds = a.rounds, K = a.K, window = a.window, bshift = a.bshift;
  const int hs = bshift - 3;  // log2 of the 8-token halves per block
  const float scale_log2 = a.scale_log2;
  float* __restrict__ part = a.part;
  auto& kst = sh.kst;
  auto& sm_o = sh.sm_o;
  auto& sm_m = sh.sm_m;
  auto& sm_l = sh.sm_l;
  if (threadIdx.x == 0) sh.arrived = 0;
  __syncthreads();  // before any request is issued: the waves of a workgroup start together

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int split_units = rounds * kAttnWaves;
  const int len_raw = a.seq_lens[bh / heads];
  const int tc_raw = RES ? 0 : a.table_count[bh];
  // The table entries head the dependent chain table -> K/V, so they are requested
  // together with the count, clamped to the row (not to the count).  Half h of unit
  // u is 8-token half 2u + h of the table, in entry (2u + h) >> hs (both halves in
  // one entry unless the blocks hold 8 tokens).
  // The entry is wave-uniform: a scalar load (through the scalar cache) keeps it out of
  // the vector memory queues that the streaming loads fill.  The table is never written
  // by the launch that reads it.
  auto load_entry = [&](int e) {
    e = __builtin_amdgcn_readfirstlane(e);
    const size_t idx = RES ? (size_t)bh * K + (e < K ? e : K - 1) : (size_t)bh * T + (e < T ? e : T - 1);
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(table))[idx];
  };
  int ent0, ent1 = -1;
  {
    const int u = sp * split_units + wave;
    ent0 = load_entry((2 * u) >> hs);
    if (hs == 0) ent1 = load_entry(2 * u + 1);
  }
  // Columns past the group repeat the last query head; their results are never read.
  u32x4 qf[4];
  const int gq = col < group ? col : group - 1;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = q[((size_t)(bh * group + gq) * queries) * 16 + 4 * s + grp];
  __builtin_amdgcn_sched_barrier(0);  // both requests go out before the wait for the entry

  // No early exit for a workgroup past the table count: every entry past it is a
  // masked load (no memory access), the record it writes is never read by the merge,
  // and without the branch the requests above cannot be moved behind the count.
  const int len = clamp_len(len_raw, NB, bshift);
  const int tc = tc_raw < 0 ? 0 : (tc_raw > T ? T : tc_raw);
  const int w0 = first_window_block(len, window, bshift), nblk = num_blocks(len, bshift);

  constexpr uint32_t kHalfBytes = 8 * kHeadDim * 2;
  const uint32_t block_bytes = (uint32_t)(kHeadDim * 2) << bshift;
  const uint32_t head_bytes = (uint32_t)(POOL ? K : NB) * block_bytes;
  const size_t head_off = (size_t)bh * head_bytes;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(v + head_off, head_bytes);
  __amdgpu_buffer_rsrc_t rk_ring = rk, rv_ring = rv;
  if (POOL) {
    const uint32_t ring_bytes = (uint32_t)a.WB * block_bytes;
    rk_ring = head_rsrc(a.ring_k + (size_t)bh * ring_bytes, ring_bytes);
    rv_ring = head_rsrc(a.ring_v + (size_t)bh * ring_bytes, ring_bytes);
  }

  float m_run = -INFINITY;  // running max of scale*log2(e)*q.k for query head `col`
  float l_run = 0.f;        // this lane's share of the running sum
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int krow = 4 * (col & 3) + (col >> 2);  // token this lane feeds as an MFMA row

  int rd = 0;
  do {  // rounds >= 1: a do-while keeps the loads above where they are issued
    const int u = sp * split_units + rd * kAttnWaves + wave;
    const int e0 = (2 * u) >> hs, e1 = (2 * u + 1) >> hs;
    if (rd > 0) {
      ent0 = load_entry(e0);
      if (hs == 0) ent1 = load_entry(e1);
    }
    // Half h: its 8-token sub-block id8[h] in the head's token order (-1: nothing to
    // read), the byte offset of this lane's first chunk, and the buffers it is in.
    int id8[2];
    uint32_t off[2];
    __amdgpu_buffer_rsrc_t rk_h[2], rv_h[2];
    auto resolve = [&](int h, int e, int id) {
      if (RES) {
        if (e < K) {
          if (id >= w0) id = -1;  // inside the window: attended as a window block
        } else {
          id = e - K < nblk - w0 ? w0 + (e - K) : -1;
        }
      } else if (e >= tc) {
        id = -1;
      }
      if (id < 0 || id >= NB || (id << bshift) >= len) id = -1;
      rk_h[h] = rk;
      rv_h[h] = rv;
      int phys = id;  // where the block sits: its logical index in the full cache
      if (POOL) {     // ... or its pool slot, or its ring slot (all wave-uniform)
        id = __builtin_amdgcn_readfirstlane(id);
        const bool in_pool = __builtin_amdgcn_readfirstlane(e) < K;
        phys = in_pool ? e : id % a.WB;
        if (!in_pool) {
          rk_h[h] = rk_ring;
          rv_h[h] = rv_ring;
        }
      }
      const int sub = (2 * u + h) & ((1 << hs) - 1);
      int i8 = id < 0 ? -1 : (id << hs) + sub;
      if (i8 * 8 >= len) i8 = -1;  // the half lies past the sequence
      id8[h] = i8;
      off[h] = i8 < 0 ? kOffMasked : (uint32_t)((phys << hs) + sub) * kHalfBytes + lane * 16;
    };
    resolve(0, e0, ent0);
    if (hs == 0) {  // 8-token blocks: the second half is the next entry
      resolve(1, e1, ent1);
    } else {        // the next 8 tokens of the same block
      int i8 = id8[0] < 0 ? -1 : id8[0] + 1;
      if (i8 * 8 >= len) i8 = -1;
      id8[1] = i8;
      off[1] = i8 < 0 ? kOffMasked : off[0] + kHalfBytes;
      rk_h[1] = rk_h[0];
      rv_h[1] = rv_h[0];
    }
    u32x4 kr[4], vf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kr[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk_h[s >> 1], off[s >> 1] + 1024 * (s & 1), 0, kNtAux));
#pragma unroll
    for (int s = 0; s < 4; ++s)
      vf[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv_h[s >> 1], off[s >> 1] + 1024 * (s & 1), 0, kNtAux));
    // Stage K: token 4s + grp, chunk col.
#pragma unroll
    for (int s = 0; s < 4; ++s) kst[wave][(4 * s + grp) * kKRow + col] = kr[s];
    __builtin_amdgcn_wave_barrier();
    u32x4 kf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[s] = kst[wave][krow * kKRow + 4 * s + grp];
    __builtin_amdgcn_wave_barrier();
    floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), st, 0, 0, 0);
    // st[r] = q[col] . k[token 4r + grp]
    float p[4];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = id8[r >> 1] >= 0 && id8[r >> 1] * 8 + 4 * (r & 1) + grp < len;
      p[r] = ok ? st[r] * scale_log2 : -INFINITY;
      bm = fmaxf(bm, p[r]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float m_new = fmaxf(m_run, bm);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;  // no valid token yet: all weights 0
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    // hi = bf16(p) and lo = bf16(p - hi) carry p to about 2^-17 relative; the running
    // sum adds the fp32 values.
    uint32_t hw[2], lw[2];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(p[r] - m_ref);
      const float p1 = __builtin_amdgcn_exp2f(p[r + 1] - m_ref);
      psum += p0 + p1;
      const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
      const __bf16 l0 = (__bf16)(p0 - (float)h0), l1 = (__bf16)(p1 - (float)h1);
      hw[r / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lw[r / 2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] *= alpha;
    // V rows of tokens past the sequence are zeroed: their probability is 0, but the
    // memory behind them need not hold finite values (masked blocks read zeros).
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (id8[s >> 1] * 8 + 4 * (s & 1) + grp >= len) vf[s] = u32x4{0u, 0u, 0u, 0u};
    }
    const bf16x4_bits pb_hi = __builtin_bit_cast(bf16x4_bits, (uint64_t)hw[0] | ((uint64_t)hw[1] << 32));
    const bf16x4_bits pb_lo = __builtin_bit_cast(bf16x4_bits, (uint64_t)lw[0] | ((uint64_t)lw[1] << 32));
    // Tile t: lane supplies head dim 8*col + t of tokens 4e + grp (e = 0..3), the same
    // tokens whose probabilities it holds.
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int w = t >> 1;
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
      const uint32_t a0 = __builtin_amdgcn_perm(vf[1][w], vf[0][w], sel);
      const uint32_t a1 = __builtin_amdgcn_perm(vf[3][w], vf[2][w], sel);
      const bf16x4_bits va = __builtin_bit_cast(bf16x4_bits, (uint64_t)a0 | ((uint64_t)a1 << 32));
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_hi, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_lo, o[t], 0, 0, 0);
    }
  } while (++rd < rounds);

  // Publish this wave's partial.  o[t][r] holds head dim 32*grp + 8r + t of query head col.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (col < GP) {
    if (grp == 0) {
      sm_m[wave][col] = m_run;
      sm_l[wave][col] = l_run;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int t = 0; t < 8; ++t) sm_o[wave][col][32 * grp + 8 * r + t] = o[t][r];
    }
  }
  int before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(&sh.arrived, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before != kAttnWaves - 1) return;  // another wave finishes the workgroup

  // Last wave: combine the four partials into the split's record.
  float* rec0 = part + ((size_t)bh * nsplit + sp) * group * kRec;
  for (int idx = lane; idx < group * (kHeadDim / 4); idx += 64) {
    const int g = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) mx = fmaxf(mx, sm_m[w][g]);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][g] - mx);
        acc += f * *(const floatx4*)&sm_o[w][g][4 * d4];
        lsum += f * sm_l[w][g];
      }
    }
    float* rec = rec0 + g * kRec;
    *(floatx4*)(rec + 4 * d4) = acc;
    if (d4 == 0) {
      rec[kHeadDim + 0] = mx;
      rec[kHeadDim + 1] = lsum;
    }
  }
}

// One workgroup per (sequence, KV head, query head).  Every wave
// loads the (max, sum) of all splits (lane s holds splits s, s + 64, ...) and
// derives the same weights with DPP wave reductions; wave w of NWV adds the outputs
// of splits w, w + NWV, ... (lane l: head dims 2l and 2l + 1), sixteen loads in flight
// per batch, the first batch requested together with the (max, sum) values; the
// partial sums meet in LDS.
constexpr int kMergeBatch = 16;
typedef float float2v __attribute__((ext_vector_type(2)));
template <int NWV>
struct MergeShared {
  float2v acc[NWV][64];
};

// Query head `bhg` = (sequence, KV head) * group + g, merged by the NWV waves of the
// calling workgroup.  Every thread of the workgroup calls it.
template <int NWV>
__device__ __attribute__((always_inline)) void attn_merge_wg(int bhg, MergeShared<NWV>& sh,
                                                             const float* __restrict__ part,
                                                             int group, int nsplit,
                                                             float* __restrict__ out,
                                                             float* __restrict__ lse) {
  constexpr int kMergeWaves = NWV;
  auto& sm_acc = sh.acc;
  const int bh = bhg / group, g = bhg % group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Every split writes its record; splits past the table hold max -inf, sum 0 and a
  // zero output, so the merge takes all of them and needs no table count.
  const float* rec = part + ((size_t)bh * nsplit * group + g) * kRec;  // split s: + s * stride
  const size_t stride = (size_t)group * kRec;
  const size_t stride2 = stride / 2;
  const float2v* po = (const float2v*)rec + lane;

  float mloc[kAttnMaxSplits / 64], lloc[kAttnMaxSplits / 64];
#pragma unroll
  for (int c = 0; c < kAttnMaxSplits / 64; ++c) {
    const int s = c * 64 + lane;
    const int sc = s < nsplit ? s : 0;
    mloc[c] = rec[sc * stride + kHeadDim + 0];
    lloc[c] = rec[sc * stride + kHeadDim + 1];
  }
  float2v x[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const int s = wave + kMergeWaves * u;
    x[u] = po[(size_t)(s < nsplit ? s : 0) * stride2];
  }
  const int nvalid = nsplit;  // <= kAttnMaxSplits

  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < kAttnMaxSplits / 64; ++c) {
    if (c * 64 + lane >= nvalid) mloc[c] = -INFINITY;
    m = fmaxf(m, mloc[c]);
  }
  const float mx = wave_max_f32(m);
  float wl = 0.f;
  float wloc[kAttnMaxSplits / 64];
#pragma unroll
  for (int c = 0; c < kAttnMaxSplits / 64; ++c) {
    wloc[c] = (mx == -INFINITY || c * 64 + lane >= nvalid) ? 0.f : __builtin_amdgcn_exp2f(mloc[c] - mx);
    wl += wloc[c] * lloc[c];
  }
  const float sum = wave_sum_f32(wl);
  // Weight of split s (wave-uniform s): lane s % 64 of wloc[s / 64].
  auto weight = [&](int s) {
    const int c = s >> 6;
    const float w = c == 0 ? wloc[0] : (c == 1 ? wloc[1] : (c == 2 ? wloc[2] : wloc[3]));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s & 63));
  };
  float2v acc = {0.f, 0.f};
  for (int s0 = wave;; s0 += kMergeWaves * kMergeBatch) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + kMergeWaves * u;
      if (s < nvalid) acc += weight(s) * x[u];
    }
    const int s1 = s0 + kMergeWaves * kMergeBatch;
    if (s1 >= nvalid) break;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s1 + kMergeWaves * u;
      x[u] = po[(size_t)(s < nsplit ? s : 0) * stride2];
    }
  }
  sm_acc[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) acc += sm_acc[w][lane];
  const bool any = mx != -INFINITY && sum > 0.f;
  float2v* o2 = (float2v*)(out + ((size_t)bh * group + g) * kHeadDim) + lane;
  *o2 = any ? acc / sum : float2v{0.f, 0.f};
  if (lse != nullptr && lane == 0) lse[(size_t)bh * group + g] = any ? (mx + __log2f(sum)) * kLn2 : -INFINITY;
}

// Query head `bhg` merged by the calling wave alone, for at most kMergeBatch splits:
// every split's (max, sum) and output requested at once, no LDS.  With few splits per
// head (many heads), a workgroup's waves take one query head each, instead of all
// the waves sharing one head's few splits.  Every lane of the wave calls it.
constexpr int kMergeWaveSplits = kMergeBatch;
__device__ __attribute__((always_inline)) void attn_merge_wave(int bhg, const float* __restrict__ part,
                                                               int group, int nsplit,
                                                               float* __restrict__ out,
                                                               float* __restrict__ lse) {
  const int bh = bhg / group, g = bhg % group;
  const int lane = threadIdx.x & 63;
  const float* rec = part + ((size_t)bh * nsplit * group + g) * kRec;  // split s: + s * stride
  const size_t stride = (size_t)group * kRec;
  const int sl = lane < nsplit ? lane : 0;
  const float m_l = rec[sl * stride + kHeadDim + 0];
  const float l_l = rec[sl * stride + kHeadDim + 1];
  float2v x[kMergeWaveSplits];
#pragma unroll
  for (int u = 0; u < kMergeWaveSplits; ++u)
    x[u] = *((const float2v*)(rec + (size_t)(u < nsplit ? u : 0) * stride) + lane);
  const float mx = wave_max_f32(lane < nsplit ? m_l : -INFINITY);
  const float w = (mx == -INFINITY || lane >= nsplit) ? 0.f : __builtin_amdgcn_exp2f(m_l - mx);
  const float sum = wave_sum_f32(w * (lane < nsplit ? l_l : 0.f));
  float2v acc = {0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeWaveSplits; ++u) {
    if (u < nsplit) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u)) * x[u];
  }
  const bool any = mx != -INFINITY && sum > 0.f;
  float2v* o2 = (float2v*)(out + ((size_t)bh * group + g) * kHeadDim) + lane;
  *o2 = any ? acc / sum : float2v{0.f, 0.f};
  if (lse != nullptr && lane == 0) lse[(size_t)bh * group + g] = any ? (mx + __log2f(sum)) * kLn2 : -INFINITY;
}

// Workgroups of the merge for `n_qh` query heads: one per query head, or, with at most
// kMergeWaveSplits splits, one per `waves` query heads.
__host__ __device__ inline int merge_workgroups(int n_qh, int nsplit, int waves) {
  return nsplit <= kMergeWaveSplits ? (n_qh + waves - 1) / waves : n_qh;
}

// Query head of wave `wave` in merge workgroup `wg` of the one-head-per-wave merge
// (-1: none).  When a KV head's query heads fill whole workgroups, those of KV head h
// run on XCD h % 8, where its splits ran when they were placed by XCD.
__device__ inline int merge_wave_head(int wg, int wave, int waves, int group, int n_qh) {
  if (group % waves == 0) {
    int x, head;
    xcd_item(wg, group / waves, n_qh / group, true, x, head);
    return head * group + x * waves + wave;
  }
  const int bhg = wg * waves + wave;
  return bhg < n_qh ? bhg : -1;
}

// Host side: the argument block of the split kernels for `d` and split `s`.
inline AttnArgs attn_args(const Dims& d, const AttnSplit& s, const void* q, const void* k, const void* v,
                   const int32_t* table, const int32_t* table_count, int table_stride,
                   const int32_t* seq_lens, float scale, void* ws) {
  AttnArgs a;
  a.q = (const u32x4*)q;
  a.k = (const char*)k;
  a.v = (const char*)v;
  a.table = table;
  a.table_count = table_count;
  a.T = table_stride;
  a.seq_lens = seq_lens;
  a.scale_log2 = scale * kLog2e;
  a.part = (float*)ws;
  a.heads = d.heads;
  a.group = d.group;
  a.queries = d.queries;
  a.NB = d.max_blocks;
  a.nsplit = s.num_splits;
  a.rounds = s.rounds;
  a.K = d.top_k;
  a.window = d.window;
  a.bshift = d.bshift;
  a.ring_k = nullptr;
  a.ring_v = nullptr;
  a.WB = d.table_stride - d.top_k;
  return a;
}

}  // namespace oasis
