// Sparse decode attention over the head-wise block table on gfx950.
//
// Foreground attention of the target queries over the sparse working set:
// the resident (selected) blocks plus the local window (xllm-io review of
// OasisKV, section three: training flow step 3 and the architecture figure;
// legiblepapers.com summary).  Every KV head has its own table of logical
// block ids (xllm-io review, section four, Head-wise Mapping).
//
// Split-K over table entries: each workgroup takes a run of table entries of
// one (sequence, KV head); each of its four waves handles kAttnBlocksPerWave
// 16-token blocks per round with an online softmax, the waves merge in LDS,
// and the workgroup writes one (max, sum, unnormalised output) partial per
// query head.  A second kernel merges the partials of a head by log-sum-exp
// weights; the kernel boundary, not a device-scope fence, makes the partials
// visible (on this multi-XCD part a device-scope fence writes back and
// invalidates the whole L2).
//
// Per block, per wave (G <= 16 query heads padded to 16 MFMA columns):
//   S^T = K (16 tokens x 128) . q^T          4 x v_mfma_f32_16x16x32_bf16
//   O^T += V^T (128 x 16 tokens) . P^T        32 x v_mfma_f32_16x16x4_f32
// bf16 K and q multiply exactly; P stays fp32 and V widens exactly to fp32, so
// the result carries only fp32 accumulation rounding.  The token order inside
// the PV contraction is chosen so that each lane feeds the probabilities it
// computed itself (no cross-lane exchange), and the head-dim order inside an
// output tile is interleaved so that each lane feeds one element of a 16-byte
// V load it already holds.  Lane l ends up owning query head l%16 and head
// dims [32*(l/16), 32*(l/16)+32), i.e. 128 contiguous output bytes.
#include "common.h"
#include "launch.h"

namespace oasis {

constexpr int kAttnWaves = 4;
constexpr int kAttnBlocksPerWave = 2;                          // blocks in flight per wave
constexpr int kAttnBlocksPerRound = kAttnWaves * kAttnBlocksPerWave;
constexpr int kAttnMaxSplits = 64;                             // partials per head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

AttnSplit attn_split(int table_stride) {
  // Enough rounds per workgroup that no head has more than kAttnMaxSplits partials.
  const int rounds_needed = (table_stride + kAttnBlocksPerRound - 1) / kAttnBlocksPerRound;
  const int rounds = (rounds_needed + kAttnMaxSplits - 1) / kAttnMaxSplits;
  AttnSplit s;
  s.blocks_per_split = rounds * kAttnBlocksPerRound;
  s.num_splits = (table_stride + s.blocks_per_split - 1) / s.blocks_per_split;
  return s;
}

// Workspace: the partial outputs, then (max, sum) pairs.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_workspace_bytes(const Dims& d, int table_stride) {
  const AttnSplit s = attn_split(table_stride);
  const size_t parts = (size_t)d.batch * d.heads * s.num_splits * d.group;
  return align256(parts * (kHeadDim + 2) * sizeof(float));
}

__device__ inline float bf16_elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// One workgroup: `rounds` rounds of kAttnBlocksPerRound table entries of one head.
__global__ __launch_bounds__(256) void attn_split_kernel(
    const u32x4* __restrict__ q, const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int32_t* __restrict__ table, const int32_t* __restrict__ table_count, int T,
    const int32_t* __restrict__ seq_lens, float scale_log2, float* __restrict__ part_o,
    float* __restrict__ part_ml, int heads, int group, int queries, int NB, int nsplit, int rounds) {
  __shared__ float sm_m[kAttnWaves][16];
  __shared__ float sm_l[kAttnWaves][16];
  __shared__ float sm_o[kAttnWaves][16][kHeadDim + 4];

  const int bh = blockIdx.y, sp = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int len = clamp_len(seq_lens[bh / heads], NB);
  int tc = table_count[bh];
  tc = tc < 0 ? 0 : (tc > T ? T : tc);
  const int split_blocks = rounds * kAttnBlocksPerRound;
  if (sp * split_blocks >= tc) return;  // the merge reads only splits below ceil(tc / split_blocks)

  u32x4 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = (col < group) ? q[((size_t)(bh * group + col) * queries) * 16 + 4 * s + grp]
                          : u32x4{0u, 0u, 0u, 0u};
  }
  float m_run = -INFINITY;  // running max of scale*log2(e)*q.k for query head `col`
  float l_run = 0.f;        // this lane's share of the running sum
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int rd = 0; rd < rounds; ++rd) {
    const int e0 = sp * split_blocks + rd * kAttnBlocksPerRound + wave * kAttnBlocksPerWave;
    if (e0 >= tc) break;  // uniform across the wave
    u32x4 kf[kAttnBlocksPerWave][4], vf[kAttnBlocksPerWave][4];
    int blk[kAttnBlocksPerWave];
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
      const int e = e0 + a;
      int id = (e < tc) ? table[(size_t)bh * T + e] : -1;
      if (id < 0 || id >= NB || id * kBlock >= len) id = -1;
      blk[a] = id;
      const size_t base = ((size_t)bh * NB + (id < 0 ? 0 : id)) * (kBlock * 16);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // K: token `col`, 16-byte chunk 4s + grp.  V: token 4*grp + s, chunk `col`.
        kf[a][s] = (id >= 0) ? k[base + col * 16 + 4 * s + grp] : u32x4{0u, 0u, 0u, 0u};
        vf[a][s] = (id >= 0) ? v[base + (4 * grp + s) * 16 + col] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
      if (blk[a] < 0) continue;  // uniform across the wave
      floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[a][s]), as_bf16x8(qf[s]), st, 0, 0, 0);
      }
      // st[i] = q[col] . k[token 4*grp + i]
      const int tok0 = blk[a] * kBlock + 4 * grp;
      float p[4];
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (tok0 + i < len) ? st[i] * scale_log2 : -INFINITY;
        bm = fmaxf(bm, p[i]);
      }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run, bm);  // finite: the block holds a valid token
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(p[i] - m_new);
        psum += p[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_elem(vf[a][s], t), p[s], o[t], 0, 0, 0);
        }
      }
    }
  }

  // Merge the four waves in LDS.  o[t][r] holds head dim 32*grp + 8r + t of query head col.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (grp == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int t = 0; t < 8; ++t) sm_o[wave][col][32 * grp + 8 * r + t] = o[t][r];
  }
  __syncthreads();
  const size_t part = (size_t)bh * nsplit + sp;
  for (int idx = threadIdx.x; idx < group * kHeadDim; idx += blockDim.x) {
    const int g = idx / kHeadDim, dd = idx % kHeadDim;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) mx = fmaxf(mx, sm_m[w][g]);
    float acc = 0.f, lsum = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][g] - mx);
        acc += f * sm_o[w][g][dd];
        lsum += f * sm_l[w][g];
      }
    }
    part_o[(part * group + g) * kHeadDim + dd] = acc;
    if (dd == 0) {
      part_ml[(part * group + g) * 2 + 0] = mx;
      part_ml[(part * group + g) * 2 + 1] = lsum;
    }
  }
}

// One workgroup per head.  Wave g handles query head g (and g + 4, ...): lane s holds
// split s's (max, sum) so the weights come from two DPP wave reductions; then
// every thread sums its float4 of the output over the splits with all loads issued
// before the first add.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         const int32_t* __restrict__ table_count,
                                                         int T, int group, int nsplit,
                                                         int split_blocks, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ float sm_w[kAttnMaxSplits][16];
  __shared__ float sm_mx[16], sm_sum[16];
  const int bh = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int tc = table_count[bh];
  tc = tc < 0 ? 0 : (tc > T ? T : tc);
  const int nvalid = (tc + split_blocks - 1) / split_blocks;  // <= nsplit <= kAttnMaxSplits
  const size_t part0 = (size_t)bh * nsplit;
  for (int g = wave; g < group; g += kAttnWaves) {
    float m = -INFINITY, l = 0.f;
    if (lane < nvalid) {
      m = part_ml[((part0 + lane) * group + g) * 2 + 0];
      l = part_ml[((part0 + lane) * group + g) * 2 + 1];
    }
    const float mx = wave_max_f32(m);
    const float w = (mx == -INFINITY || lane >= nvalid) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
    const float sum = wave_sum_f32(w * l);
    if (lane < nvalid) sm_w[lane][g] = w;
    if (lane == 0) {
      sm_mx[g] = mx;
      sm_sum[g] = sum;
    }
  }
  __syncthreads();
  const floatx4* po = (const floatx4*)part_o;
  for (int idx = threadIdx.x; idx < group * (kHeadDim / 4); idx += blockDim.x) {
    const int g = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= nvalid; s += 8) {
      floatx4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = po[((part0 + s + u) * group + g) * (kHeadDim / 4) + d4];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += sm_w[s + u][g] * x[u];
    }
    for (; s < nvalid; ++s) acc += sm_w[s][g] * po[((part0 + s) * group + g) * (kHeadDim / 4) + d4];
    const float sum = sm_sum[g];
    const bool any = sm_mx[g] != -INFINITY && sum > 0.f;
    floatx4* o4 = (floatx4*)(out + ((size_t)bh * group + g) * kHeadDim);
    o4[d4] = any ? acc / sum : floatx4{0.f, 0.f, 0.f, 0.f};
    if (lse != nullptr && d4 == 0) {
      lse[(size_t)bh * group + g] = any ? (sm_mx[g] + __log2f(sum)) * kLn2 : -INFINITY;
    }
  }
}

hipError_t launch_attention_split(const Dims& d, const void* q, const void* k, const void* v,
                                  const int32_t* table, const int32_t* table_count,
                                  int table_stride, const int32_t* seq_lens, float scale, void* ws,
                                  hipStream_t stream) {
  const AttnSplit s = attn_split(table_stride);
  const size_t parts = (size_t)d.batch * d.heads * s.num_splits * d.group;
  float* part_o = (float*)ws;
  float* part_ml = part_o + parts * kHeadDim;
  attn_split_kernel<<<dim3(s.num_splits, d.batch * d.heads), dim3(64 * kAttnWaves), 0, stream>>>(
      (const u32x4*)q, (const u32x4*)k, (const u32x4*)v, table, table_count, table_stride, seq_lens,
      scale * kLog2e, part_o, part_ml, d.heads, d.group, d.queries, d.max_blocks, s.num_splits,
      s.blocks_per_split / kAttnBlocksPerRound);
  return hipGetLastError();
}

hipError_t launch_attention_merge(const Dims& d, const int32_t* table_count, int table_stride,
                                  float* out, float* lse, const void* ws, hipStream_t stream) {
  const AttnSplit s = attn_split(table_stride);
  const size_t parts = (size_t)d.batch * d.heads * s.num_splits * d.group;
  const float* part_o = (const float*)ws;
  const float* part_ml = part_o + parts * kHeadDim;
  attn_merge_kernel<<<dim3(d.batch * d.heads), dim3(64 * kAttnWaves), 0, stream>>>(
      part_o, part_ml, table_count, table_stride, d.group, s.num_splits, s.blocks_per_split, out, lse);
  return hipGetLastError();
}

hipError_t launch_attention(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* table, const int32_t* table_count, int table_stride,
                            const int32_t* seq_lens, float scale, float* out, float* lse, void* ws,
                            hipStream_t stream) {
  hipError_t err = launch_attention_split(d, q, k, v, table, table_count, table_stride, seq_lens,
                                          scale, ws, stream);
  if (err != hipSuccess) return err;
  return launch_attention_merge(d, table_count, table_stride, out, lse, ws, stream);
}

}  // namespace oasis
