// Sparse decode attention over the head-wise block table on gfx950.
//
// Foreground attention of the target queries over the sparse working set:
// the resident (selected) blocks plus the local window (xllm-io review of
// OasisKV, section three: training flow step 3 and the architecture figure;
// legiblepapers.com summary).  Every KV head has its own table of logical
// block ids (xllm-io review, section four, Head-wise Mapping).
//
// The work is a gather of 8 KB per table entry (16 tokens of K and V), and on
// this part a gather finishes soonest when each wave fetches as little as
// possible and the whole table is requested at once: one 16-token block per wave
// and round, four waves per workgroup, a workgroup per four table entries of a
// head (more rounds only when a head has over 1024 entries).  K is requested
// before V, so the QK product and the softmax run while V is in flight; the
// waves merge in LDS and each workgroup writes one (max, sum, unnormalised
// output) partial per query head; a second kernel merges the partials of a
// head by log-sum-exp weights (the kernel boundary, not a device-scope fence,
// makes them visible: on this multi-XCD part such a fence writes back and
// invalidates the whole L2).  K and V are read with buffer loads through a
// per-head resource whose range check turns a masked load (past the table, an
// invalid id, a block past the sequence) into zeros without a memory access.
//
// Per block, per wave (G <= 16 query heads padded to 16 MFMA columns):
//   S^T = K (16 tokens x 128) . q^T           4 x v_mfma_f32_16x16x32_bf16
//   O^T += V^T (128 x 16 tokens) . P^T        2 x 8 x v_mfma_f32_16x16x16_bf16
// bf16 K and q multiply exactly.  Each fp32 probability p enters the PV product
// as two bf16 terms, bf16(p) and bf16(p - bf16(p)), which carry p to about 2^-17
// relative at twice the (small) cost of one bf16 product.  The token order
// inside the PV contraction is chosen so that each lane feeds the probabilities
// it computed itself (no cross-lane exchange), and the head-dim order inside an
// output tile is interleaved so that each lane feeds one element of a 16-byte V
// load it already holds.  Lane l ends up owning query head l%16 and head dims
// [32*(l/16), 32*(l/16)+32), i.e. 128 contiguous output bytes.
#include "common.h"
#include "launch.h"

namespace oasis {



constexpr int kAttnWaves = 4;                 // one table entry per wave and round
constexpr int kAttnMaxSplits = 256;           // partials per head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short bf16x4_bits __attribute__((ext_vector_type(4)));

AttnSplit attn_split(const Dims&, int table_stride) {
  // Rounds per workgroup: enough that no head has more than kAttnMaxSplits partials.
  const int groups = (table_stride + kAttnWaves - 1) / kAttnWaves;
  AttnSplit s;
  s.rounds = (groups + kAttnMaxSplits - 1) / kAttnMaxSplits;
  if (s.rounds < 1) s.rounds = 1;
  s.num_splits = (table_stride + kAttnWaves * s.rounds - 1) / (kAttnWaves * s.rounds);
  if (s.num_splits < 1) s.num_splits = 1;
  return s;
}

// Workspace: one record per (sequence, KV head, split, query head): the unnormalised
// output (128 floats), the running max (log2 units), the sum, and padding to 16
// bytes.  Records of one (sequence, KV head) are contiguous, so a run of sequences
// owns a contiguous slice of the workspace.
constexpr int kRec = kHeadDim + 4;
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_workspace_bytes(const Dims& d, int table_stride) {
  const AttnSplit s = attn_split(d, table_stride);
  return align256((size_t)d.batch * d.heads * s.num_splits * d.group * kRec * sizeof(float));
}

size_t attn_workspace_bytes_per_sequence(const Dims& d, int table_stride) {
  const AttnSplit s = attn_split(d, table_stride);
  return (size_t)d.heads * s.num_splits * d.group * kRec * sizeof(float);
}

// Buffer resource over one head's K or V blocks; an offset at or past `bytes` reads
// zeros and touches no memory.
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOffMasked = 0x80000000u;
constexpr int kNtAux = 2;  // non-temporal: K and V are read once

// K and V blocks are read with fully contiguous 1 KB wave loads (instruction s of
// a block covers tokens 4s..4s+3): lane l holds token 4s + l/16, 16-byte chunk
// l%16.  That is already the layout the PV product wants for V.  For QK, lane l
// must supply one token's chunks, so K goes through LDS (rows padded to 272
// bytes, conflict-free) and is read back with MFMA row i holding token
// 4*(i%4) + i/4; the scores then come out with lane l owning exactly the tokens
// 4r + l/16 whose V rows it loaded.
constexpr int kKRow = kHeadDim * 2 / 16 + 1;  // padded LDS row of one K token, in 16-byte chunks

#ifndef OASIS_ATTN_MIN_WAVES
#define OASIS_ATTN_MIN_WAVES 4  // <= 128 VGPRs: four waves per SIMD
#endif
// GP: query heads per KV head rounded up to 4, 8 or 16 (sizes the LDS partials).
template <int GP>
__global__ __launch_bounds__(256, OASIS_ATTN_MIN_WAVES) void attn_split_kernel(
    const u32x4* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v,
    const int32_t* __restrict__ table, const int32_t* __restrict__ table_count, int T,
    const int32_t* __restrict__ seq_lens, float scale_log2, float* __restrict__ part,
    int heads, int group, int queries, int NB, int nsplit, int rounds) {
  __shared__ u32x4 kst[kAttnWaves][kBlock * kKRow];  // per-wave K staging
  // Per-wave partials: the waves merge without a barrier; the last one to finish
  // combines them and writes the record, the others end as soon as they have
  // published theirs (freeing their slots for waves of other workgroups).
  __shared__ alignas(16) float sm_o[kAttnWaves][GP][kHeadDim + 4];
  __shared__ float sm_m[kAttnWaves][GP];
  __shared__ float sm_l[kAttnWaves][GP];
  __shared__ int arrived;
  if (threadIdx.x == 0) arrived = 0;
  __syncthreads();  // before any request is issued: the waves of a workgroup start together

  const int bh = blockIdx.y, sp = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int split_entries = rounds * kAttnWaves;
  const int len_raw = seq_lens[bh / heads];
  const int tc_raw = table_count[bh];
  // The table entry heads the dependent chain table -> K/V, so it is requested
  // together with the count, clamped to the row (not to the count).
  int ent;
  {
    const int e = sp * split_entries + wave;
    ent = table[(size_t)bh * T + (e < T ? e : T - 1)];
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
  const int len = clamp_len(len_raw, NB);
  const int tc = tc_raw < 0 ? 0 : (tc_raw > T ? T : tc_raw);

  const uint32_t head_bytes = (uint32_t)NB * (kBlock * kHeadDim * 2);
  const size_t head_off = (size_t)bh * head_bytes;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(v + head_off, head_bytes);

  float m_run = -INFINITY;  // running max of scale*log2(e)*q.k for query head `col`
  float l_run = 0.f;        // this lane's share of the running sum
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int krow = 4 * (col & 3) + (col >> 2);  // token this lane feeds as an MFMA row

  int rd = 0;
  do {  // rounds >= 1: a do-while keeps the loads above where they are issued
    const int e = sp * split_entries + rd * kAttnWaves + wave;
    if (rd > 0) ent = table[(size_t)bh * T + (e < T ? e : T - 1)];
    int id = ent;
    if (e >= tc || id < 0 || id >= NB || id * kBlock >= len) id = -1;
    const uint32_t off = id < 0 ? kOffMasked : (uint32_t)id * (kBlock * kHeadDim * 2) + lane * 16;
    u32x4 kr[4], vf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kr[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off + 1024 * s, 0, kNtAux));
#pragma unroll
    for (int s = 0; s < 4; ++s)
      vf[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off + 1024 * s, 0, kNtAux));
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
      const bool ok = id >= 0 && id * kBlock + 4 * r + grp < len;
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
      if (id * kBlock + 4 * s + grp >= len) vf[s] = u32x4{0u, 0u, 0u, 0u};
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
    before = __hip_atomic_fetch_add(&arrived, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
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

// One workgroup of four waves per (sequence, KV head, query head).  Every wave
// loads the (max, sum) of all splits (lane s holds splits s, s + 64, ...) and
// derives the same weights with DPP wave reductions; wave w adds the outputs of
// splits w, w + 4, ... (lane l: head dims 2l and 2l + 1), sixteen loads in flight
// per batch, the first batch requested together with the (max, sum) values; the
// four partial sums meet in LDS.
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 16;
typedef float float2v __attribute__((ext_vector_type(2)));
__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ table_count, int T, int group,
    int nsplit, int split_entries, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float2v sm_acc[kMergeWaves][64];
  const int bh = blockIdx.x / group, g = blockIdx.x % group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Loads are clamped to the split count, not to the table count (every split writes
  // its record), so that they need not wait for the count.
  const int tc_raw = table_count[bh];
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
  const int tc = tc_raw < 0 ? 0 : (tc_raw > T ? T : tc_raw);
  int nvalid = (tc + split_entries - 1) / split_entries;
  nvalid = nvalid < nsplit ? nvalid : nsplit;  // <= kAttnMaxSplits

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

hipError_t launch_attention_split(const Dims& d, const AttnSplit& s, const void* q, const void* k,
                                  const void* v, const int32_t* table, const int32_t* table_count,
                                  int table_stride, const int32_t* seq_lens, float scale, void* ws,
                                  hipStream_t stream) {
  const dim3 grid(s.num_splits, d.batch * d.heads), block(64 * kAttnWaves);
#define OASIS_ATTN_ARGS                                                                           \
  (const u32x4*)q, (const char*)k, (const char*)v, table, table_count, table_stride, seq_lens,    \
      scale * kLog2e, (float*)ws, d.heads, d.group, d.queries, d.max_blocks, s.num_splits, s.rounds
  if (d.group <= 4) {
    attn_split_kernel<4><<<grid, block, 0, stream>>>(OASIS_ATTN_ARGS);
  } else if (d.group <= 8) {
    attn_split_kernel<8><<<grid, block, 0, stream>>>(OASIS_ATTN_ARGS);
  } else {
    attn_split_kernel<16><<<grid, block, 0, stream>>>(OASIS_ATTN_ARGS);
  }
#undef OASIS_ATTN_ARGS
  return hipGetLastError();
}
hipError_t launch_attention_merge(const Dims& d, const AttnSplit& s, const int32_t* table_count,
                                  int table_stride, float* out, float* lse, const void* ws,
                                  hipStream_t stream) {
  attn_merge_kernel<<<dim3(d.batch * d.heads * d.group), dim3(64 * kMergeWaves), 0, stream>>>(
      (const float*)ws, table_count, table_stride, d.group, s.num_splits, s.rounds * kAttnWaves,
      out, lse);
  return hipGetLastError();
}

hipError_t launch_attention(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* table, const int32_t* table_count, int table_stride,
                            const int32_t* seq_lens, float scale, float* out, float* lse, void* ws,
                            hipStream_t stream) {
  const AttnSplit s = attn_split(d, table_stride);
  hipError_t err = launch_attention_split(d, s, q, k, v, table, table_count, table_stride, seq_lens,
                                          scale, ws, stream);
  if (err != hipSuccess) return err;
  return launch_attention_merge(d, s, table_count, table_stride, out, lse, ws, stream);
}

}  // namespace oasis
