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
// Per pair of blocks, per wave (G <= 16 query heads padded to 16 MFMA columns):
//   S^T = K (16 tokens x 128) . q^T           2 x 4 x v_mfma_f32_16x16x32_bf16
//   O^T += V^T (128 x 32 tokens) . P^T        2 x 8 x v_mfma_f32_16x16x32_bf16
// bf16 K and q multiply exactly.  Each fp32 probability p enters the PV product
// as two bf16 terms, bf16(p) and bf16(p - bf16(p)), which carry p to about 2^-17
// relative at twice the (small) cost of one bf16 product.  (Built with
// OASIS_ATTN_PV_BF16=0, PV runs as 32 fp32 v_mfma_f32_16x16x4_f32 per block
// instead.)  The token
// order inside the PV contraction is chosen so that each lane feeds the
// probabilities it computed itself (no cross-lane exchange), and the head-dim
// order inside an output tile is interleaved so that each lane feeds one element
// of a 16-byte V load it already holds.  Lane l ends up owning query head l%16
// and head dims [32*(l/16), 32*(l/16)+32), i.e. 128 contiguous output bytes.
#include "common.h"
#include "launch.h"

namespace oasis {

#ifndef OASIS_ATTN_BLOCKS_PER_WAVE
#define OASIS_ATTN_BLOCKS_PER_WAVE 2
#endif
#ifndef OASIS_ATTN_MIN_ROUNDS
#define OASIS_ATTN_MIN_ROUNDS 1
#endif
#ifndef OASIS_ATTN_PV_BF16
#define OASIS_ATTN_PV_BF16 1
#endif
constexpr int kAttnWaves = 4;
constexpr int kAttnBlocksPerWave = OASIS_ATTN_BLOCKS_PER_WAVE;  // blocks in flight per wave
constexpr int kAttnBlocksPerRound = kAttnWaves * kAttnBlocksPerWave;
constexpr int kAttnMaxSplits = 64;                             // partials per head
static_assert(!OASIS_ATTN_PV_BF16 || kAttnBlocksPerWave % 2 == 0,
              "the bf16 PV product takes blocks in pairs");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

AttnSplit attn_split(int table_stride) {
  // Enough rounds per workgroup that no head has more than kAttnMaxSplits partials.
  const int rounds_needed = (table_stride + kAttnBlocksPerRound - 1) / kAttnBlocksPerRound;
  int rounds = (rounds_needed + kAttnMaxSplits - 1) / kAttnMaxSplits;
  if (rounds < OASIS_ATTN_MIN_ROUNDS) rounds = OASIS_ATTN_MIN_ROUNDS;
  AttnSplit s;
  s.blocks_per_split = rounds * kAttnBlocksPerRound;
  s.num_splits = (table_stride + s.blocks_per_split - 1) / s.blocks_per_split;
  return s;
}

// Workspace: one record per (sequence, KV head, split, query head): the unnormalised
// output (128 floats), the running max (log2 units), the sum, and padding to 16
// bytes.  Records of one (sequence, KV head) are contiguous, so a run of sequences
// owns a contiguous slice of the workspace.
constexpr int kRec = kHeadDim + 4;
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_workspace_bytes(const Dims& d, int table_stride) {
  const AttnSplit s = attn_split(table_stride);
  return align256((size_t)d.batch * d.heads * s.num_splits * d.group * kRec * sizeof(float));
}

size_t attn_workspace_bytes_per_sequence(const Dims& d, int table_stride) {
  const AttnSplit s = attn_split(table_stride);
  return (size_t)d.heads * s.num_splits * d.group * kRec * sizeof(float);
}

__device__ inline float bf16_elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// One workgroup: `rounds` rounds of kAttnBlocksPerRound table entries of one head.
//
// K and V blocks are read with fully contiguous 1 KB wave loads (instruction s of
// a block covers tokens 4s..4s+3): lane l holds token 4s + l/16, 16-byte chunk
// l%16.  That is already the layout the PV product wants for V.  For QK, lane l
// must supply one token's chunks, so K goes through LDS (rows padded to 272
// bytes, conflict-free) and is read back with MFMA row i holding token
// 4*(i%4) + i/4; the scores then come out with lane l owning exactly the tokens
// 4r + l/16 whose V rows it loaded.
constexpr int kKRow = kHeadDim * 2 / 16 + 1;  // padded LDS row of one K token, in 16-byte chunks

__global__ __launch_bounds__(256) void attn_split_kernel(
    const u32x4* __restrict__ q, const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int32_t* __restrict__ table, const int32_t* __restrict__ table_count, int T,
    const int32_t* __restrict__ seq_lens, float scale_log2, float* __restrict__ part,
    int heads, int group, int queries, int NB, int nsplit, int rounds) {
  __shared__ float sm_m[kAttnWaves][16];
  __shared__ float sm_l[kAttnWaves][16];
  // K staging during the rounds, then the cross-wave merge of the outputs.
  __shared__ union {
    u32x4 kst[kAttnWaves][kAttnBlocksPerWave][kBlock * kKRow];
    float o[kAttnWaves][16][kHeadDim + 4];
  } sm;

  const int bh = blockIdx.y, sp = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int len = clamp_len(seq_lens[bh / heads], NB);
  int tc = table_count[bh];
  tc = tc < 0 ? 0 : (tc > T ? T : tc);
  const int split_blocks = rounds * kAttnBlocksPerRound;
  if (sp * split_blocks >= tc) return;  // the merge reads only splits below ceil(tc / split_blocks)

  // Loads are unconditional (clamped addresses, results masked) so that no branch
  // splits them.  The first round's table entries go first: they head the
  // dependent chain table -> K/V.
  int ent[kAttnBlocksPerWave];
  {
    const int e0 = sp * split_blocks + wave * kAttnBlocksPerWave;
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
      const int e = e0 + a;
      ent[a] = table[(size_t)bh * T + (e < tc ? e : tc - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Columns past the group repeat the last query head; their results are never read.
  u32x4 qf[4];
  const int gq = col < group ? col : group - 1;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = q[((size_t)(bh * group + gq) * queries) * 16 + 4 * s + grp];

  float m_run = -INFINITY;  // running max of scale*log2(e)*q.k for query head `col`
  float l_run = 0.f;        // this lane's share of the running sum
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int krow = 4 * (col & 3) + (col >> 2);  // token this lane feeds as an MFMA row

  for (int rd = 0; rd < rounds; ++rd) {
    const int e0 = sp * split_blocks + rd * kAttnBlocksPerRound + wave * kAttnBlocksPerWave;
    if (e0 >= tc) break;  // uniform across the wave
    u32x4 kr[kAttnBlocksPerWave][4], vf[kAttnBlocksPerWave][4];
    int blk[kAttnBlocksPerWave];
    if (rd > 0) {
#pragma unroll
      for (int a = 0; a < kAttnBlocksPerWave; ++a) {
        const int e = e0 + a;
        ent[a] = table[(size_t)bh * T + (e < tc ? e : tc - 1)];
      }
    }
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
      const int e = e0 + a;
      int id = ent[a];
      if (e >= tc || id < 0 || id >= NB || id * kBlock >= len) id = -1;
      blk[a] = id;
      const size_t base = ((size_t)bh * NB + (id < 0 ? 0 : id)) * (kBlock * 16) + lane;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kr[a][s] = __builtin_nontemporal_load(k + base + 64 * s);
        vf[a][s] = __builtin_nontemporal_load(v + base + 64 * s);
      }
    }
    // Keep every load of the round ahead of the arithmetic that consumes them.
    __builtin_amdgcn_sched_barrier(0);
    // Stage K: token 4s + grp, chunk col.
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sm.kst[wave][a][(4 * s + grp) * kKRow + col] = kr[a][s];
    }
    __builtin_amdgcn_wave_barrier();
    u32x4 kf[kAttnBlocksPerWave][4];
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[a][s] = sm.kst[wave][a][krow * kKRow + 4 * s + grp];
    }
    __builtin_amdgcn_wave_barrier();
    // V rows of tokens past the sequence (or of a skipped block) are zeroed: their
    // probability is 0, but the memory behind them need not hold finite values.
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (blk[a] < 0 || blk[a] * kBlock + 4 * s + grp >= len) vf[a][s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#if OASIS_ATTN_PV_BF16
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; a += 2) {
      float p[2][4];
      float bm = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[a + h][s]), as_bf16x8(qf[s]), st,
                                                       0, 0, 0);
        }
        // st[r] = q[col] . k[token 4r + grp]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = blk[a + h] >= 0 && blk[a + h] * kBlock + 4 * r + grp < len;
          p[h][r] = ok ? st[r] * scale_log2 : -INFINITY;
          bm = fmaxf(bm, p[h][r]);
        }
      }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run, bm);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;  // no valid token yet: all weights 0
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
      // Each probability enters the bf16 PV product as two bf16 terms, hi = bf16(p)
      // and lo = bf16(p - hi), so p is carried to about 2^-17 relative; the
      // running sum adds the fp32 values.
      uint32_t hw[4], lw[4];
      float psum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(p[h][r] - m_ref);
          const float p1 = __builtin_amdgcn_exp2f(p[h][r + 1] - m_ref);
          psum += p0 + p1;
          const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
          const __bf16 l0 = (__bf16)(p0 - (float)h0), l1 = (__bf16)(p1 - (float)h1);
          hw[2 * h + r / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          lw[2 * h + r / 2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
      const u32x4 pb_hi = {hw[0], hw[1], hw[2], hw[3]};
      const u32x4 pb_lo = {lw[0], lw[1], lw[2], lw[3]};
      // Tile t: lane supplies head dim 8*col + t of tokens 4s + grp of both blocks.
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int w = t >> 1;
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
        u32x4 va;
        va[0] = __builtin_amdgcn_perm(vf[a][1][w], vf[a][0][w], sel);
        va[1] = __builtin_amdgcn_perm(vf[a][3][w], vf[a][2][w], sel);
        va[2] = __builtin_amdgcn_perm(vf[a + 1][1][w], vf[a + 1][0][w], sel);
        va[3] = __builtin_amdgcn_perm(vf[a + 1][3][w], vf[a + 1][2][w], sel);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb_hi), o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb_lo), o[t], 0, 0, 0);
      }
    }
#else
#pragma unroll
    for (int a = 0; a < kAttnBlocksPerWave; ++a) {
      floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[a][s]), as_bf16x8(qf[s]), st, 0, 0, 0);
      }
      // st[r] = q[col] . k[token 4r + grp]
      float p[4];
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = blk[a] >= 0 && blk[a] * kBlock + 4 * r + grp < len;
        p[r] = ok ? st[r] * scale_log2 : -INFINITY;
        bm = fmaxf(bm, p[r]);
      }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run, bm);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;  // no valid token yet: all weights 0
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(p[r] - m_ref);
        psum += p[r];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
      // Step s contracts tokens 4s + (lane group): V element t of this lane's row, own p[s].
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_elem(vf[a][s], t), p[s], o[t], 0, 0, 0);
        }
      }
    }
#endif
  }
  __syncthreads();  // the K staging area becomes the merge area

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
    for (int t = 0; t < 8; ++t) sm.o[wave][col][32 * grp + 8 * r + t] = o[t][r];
  }
  __syncthreads();
  float* rec0 = part + ((size_t)bh * nsplit + sp) * group * kRec;
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
        acc += f * sm.o[w][g][dd];
        lsum += f * sm_l[w][g];
      }
    }
    float* rec = rec0 + g * kRec;
    rec[dd] = acc;
    if (dd == 0) {
      rec[kHeadDim + 0] = mx;
      rec[kHeadDim + 1] = lsum;
    }
  }
}

// One workgroup per head.  Wave g handles query head g (and g + 4, ...): lane s holds
// split s's (max, sum) so the weights come from two DPP wave reductions; then
// every thread sums its float4 of the output over the splits with all loads issued
// before the first add.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part,
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
  const float* head = part + (size_t)bh * nsplit * group * kRec;
  for (int g = wave; g < group; g += kAttnWaves) {
    float m = -INFINITY, l = 0.f;
    if (lane < nvalid) {
      m = head[((size_t)lane * group + g) * kRec + kHeadDim + 0];
      l = head[((size_t)lane * group + g) * kRec + kHeadDim + 1];
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
  for (int idx = threadIdx.x; idx < group * (kHeadDim / 4); idx += blockDim.x) {
    const int g = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
    const floatx4* po = (const floatx4*)(head + (size_t)g * kRec) + d4;
    const size_t stride4 = (size_t)group * kRec / 4;  // records of consecutive splits
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= nvalid; s += 8) {
      floatx4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = po[(size_t)(s + u) * stride4];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += sm_w[s + u][g] * x[u];
    }
    for (; s < nvalid; ++s) acc += sm_w[s][g] * po[(size_t)s * stride4];
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
  attn_split_kernel<<<dim3(s.num_splits, d.batch * d.heads), dim3(64 * kAttnWaves), 0, stream>>>(
      (const u32x4*)q, (const u32x4*)k, (const u32x4*)v, table, table_count, table_stride, seq_lens,
      scale * kLog2e, (float*)ws, d.heads, d.group, d.queries, d.max_blocks, s.num_splits,
      s.blocks_per_split / kAttnBlocksPerRound);
  return hipGetLastError();
}

hipError_t launch_attention_merge(const Dims& d, const int32_t* table_count, int table_stride,
                                  float* out, float* lse, const void* ws, hipStream_t stream) {
  const AttnSplit s = attn_split(table_stride);
  attn_merge_kernel<<<dim3(d.batch * d.heads), dim3(64 * kAttnWaves), 0, stream>>>(
      (const float*)ws, table_count, table_stride, d.group, s.num_splits, s.blocks_per_split, out, lse);
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
