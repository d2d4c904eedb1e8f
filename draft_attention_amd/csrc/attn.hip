// attn.hip -- split-K flash-decoding attention for gfx950 (MI355X), used by the three attention
// entry points: the Windowed-MTP draft step (attend the occupied slots of a compact ring buffer),
// the native full-context draft step and the target's causal verification of m draft candidates
// (Windowed-MTP abstract, third and fifth sentences: the draft normally attends the whole KV cache;
// the windowed draft attends sinks plus a recent window; verification stays full attention).
//
// Kernel 1 (attn_split_kernel): one 64-lane wavefront owns one (sequence, KV head, row chunk, key
// range). The G*m query rows of a KV head are one dense operand (GQA), so both products run on the
// matrix cores:
//   S^T (16 keys x 16 rows) = K_tile (16 x d) . Q^T          v_mfma_f32_16x16x32_bf16 / 16x16x4_f32
//   O^T (16 dims x 16 rows) += V_tile^T (16 x 16 keys) . P^T  v_mfma_f32_16x16x16_bf16 / 16x16x4_f32
// With this orientation every lane of both results holds one query row (lane & 15), so the
// running max, running sum and the rescaling of O are per-lane scalars, and the softmax weights
// computed in the S^T registers are already the P^T operand of the second product: no LDS and no
// cross-lane traffic except two xor-shuffles for the row maximum.
// K rows are read straight from HBM into the operand layout (16-byte loads, 64 contiguous bytes per
// key per instruction). V rows are read with each 16-lane group streaming one key's row (256
// contiguous bytes) and are transposed in registers with v_perm_b32 into the V^T operand.
// Each wavefront leaves (o unnormalised, running max in log2 units, running sum) for its rows.
//
// Kernel 2 (merge_kernel): log-sum-exp merge of the partials of every output row:
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s o_s 2^(m_s - M) / L,  lse = (M + log2 L) ln 2.

#include <type_traits>

#include "wmtp_internal.h"

namespace wmtp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xgroup_max(float x) {
  // lanes r, r+16, r+32, r+48 hold the same query row
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float xgroup_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Two bf16 from the low (hi = false) or high halves of two dwords: (lo16(a), lo16(b)) packed with
// a in the low half.
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, bool hi) {
  return __builtin_amdgcn_perm(b, a, hi ? 0x07060302u : 0x05040100u);
}

template <int D, bool BF16>
struct Frag {
  // query-row operand of S^T = K . Q^T, per 16-row block
  static constexpr int kQRegs = BF16 ? D / 32 : D / 16;  // bf16x8 or float4 per lane
  // V: dims each lane reads per key per "set", sets per row
  static constexpr int kDpl = BF16 ? (D >= 128 ? 8 : 4) : 4;
  static constexpr int kSetDims = 16 * kDpl;
  static constexpr int kSets = D / kSetDims;
  static constexpr int kBlocks = D / 16;  // 16-dim output blocks
};

template <int D, int NR, bool BF16>
__global__ __launch_bounds__(64 * kWavesPerBlock) void attn_split_kernel(
    AttnArgs a, int n_splits, int keys_per_split, int n_chunks, int chunk_rows) {
  using F = Frag<D, BF16>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.x * kWavesPerBlock + wave;
  if (split >= n_splits) return;  // wavefront-uniform; the kernel has no workgroup barrier

  const int bhc = blockIdx.y;
  const int chunk = bhc % n_chunks;
  const int bh = bhc / n_chunks;
  const int h = bh % a.n_kv_heads;
  const int b = bh / a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int rows = G * a.m;
  const int row0 = chunk * chunk_rows;
  const int row_end = min(rows, row0 + chunk_rows);

  int n = a.seq_len[b];
  n = max(n, 0);
  n = min(n, a.limit);
  const int kb = split * keys_per_split;
  const int ke = min(kb + keys_per_split, n);

  const int r16 = lane & 15;
  const int grp = lane >> 4;

  // ---- query rows of this lane: row = row0 + rb*16 + r16 -> candidate jq, head hq
  int last_visible[NR];  // largest key index the row may attend
  bool row_ok[NR];
  const size_t kv_head_off = (size_t)(b * a.n_kv_heads + h) * (size_t)a.capacity * D;
  typedef typename std::conditional<BF16, bf16x8_t, f32x4_t>::type QVec;
  QVec qf[NR][F::kQRegs];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int row = row0 + rb * 16 + r16;
    row_ok[rb] = row < row_end;
    const int jq = row_ok[rb] ? row / G : 0;
    const int hq = h * G + (row_ok[rb] ? row % G : 0);
    last_visible[rb] = (a.mode == kModeVerify) ? (n - a.m + jq) : (n - 1);
    const size_t qoff = ((size_t)(b * a.m + jq) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int ks = 0; ks < F::kQRegs; ++ks) {
      if constexpr (BF16) {
        // dims ks*32 + grp*8 .. +7 (the same chunk the K operand uses)
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (row_ok[rb])
          raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qoff +
                                                ks * 32 + grp * 8);
        qf[rb][ks] = __builtin_bit_cast(bf16x8_t, raw);
      } else {
        // dims ks*16 + grp*4 .. +3
        float4 raw = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_ok[rb])
          raw = *reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff + ks * 16 +
                                                 grp * 4);
        qf[rb][ks] = f32x4_t{raw.x, raw.y, raw.z, raw.w};
      }
    }
  }

  const float scale_log2 = a.sm_scale * kLog2e;
  float m_run[NR], l_run[NR];
  f32x4_t o[NR][F::kBlocks];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int i = 0; i < F::kBlocks; ++i) o[rb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = kb; t0 < ke; t0 += kTileKeys) {
    const int last = ke - 1;  // >= t0
    // ---------------- S^T = K_tile . Q^T
    f32x4_t s[NR];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) s[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const int key = min(t0 + r16, last);
      if constexpr (BF16) {
        const uint4* kp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) +
                                                         kv_head_off + (size_t)key * D);
        uint4 kf[F::kQRegs];
#pragma unroll
        for (int ks = 0; ks < F::kQRegs; ++ks) kf[ks] = kp[ks * 4 + grp];
#pragma unroll
        for (int ks = 0; ks < F::kQRegs; ++ks)
#pragma unroll
          for (int rb = 0; rb < NR; ++rb)
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]),
                                                            qf[rb][ks], s[rb], 0, 0, 0);
      } else {
        const float4* kp = reinterpret_cast<const float4*>(static_cast<const float*>(a.k) +
                                                           kv_head_off + (size_t)key * D);
        float4 kf[F::kQRegs];
#pragma unroll
        for (int ks = 0; ks < F::kQRegs; ++ks) kf[ks] = kp[ks * 4 + grp];
#pragma unroll
        for (int ks = 0; ks < F::kQRegs; ++ks)
#pragma unroll
          for (int rb = 0; rb < NR; ++rb) {
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[ks].x, qf[rb][ks][0], s[rb], 0, 0, 0);
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[ks].y, qf[rb][ks][1], s[rb], 0, 0, 0);
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[ks].z, qf[rb][ks][2], s[rb], 0, 0, 0);
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[ks].w, qf[rb][ks][3], s[rb], 0, 0, 0);
          }
      }
    }

    // ---------------- online softmax; lane holds keys t0 + 4*grp + j (j = 0..3) of its row
    float p[NR][4];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
      const int vis = min(last, last_visible[rb]);
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = t0 + 4 * grp + j;
        sc[j] = (key <= vis) ? s[rb][j] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      mx = xgroup_max(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[rb][j] = __builtin_amdgcn_exp2f(sc[j] - m_use);
        psum += p[rb][j];
      }
      l_run[rb] = l_run[rb] * alpha + psum;
      m_run[rb] = m_new;
#pragma unroll
      for (int i = 0; i < F::kBlocks; ++i) o[rb][i] *= alpha;
    }

    // ---------------- O^T += V_tile^T . P^T
    if constexpr (BF16) {
      s16x4_t pop[NR];
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        bf16x4_t pb = __builtin_convertvector(f32x4_t{p[rb][0], p[rb][1], p[rb][2], p[rb][3]},
                                              bf16x4_t);
        pop[rb] = __builtin_bit_cast(s16x4_t, pb);
      }
      // lane (r16, grp) reads keys t0 + 4*grp + t, dims set*kSetDims + r16*kDpl .. + kDpl - 1
      constexpr int kWords = F::kDpl / 2;  // dwords per key per set
      uint32_t vw[4][F::kSets][kWords];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int key = min(t0 + 4 * grp + t, last);
        const uint16_t* vp =
            static_cast<const uint16_t*>(a.v) + kv_head_off + (size_t)key * D + r16 * F::kDpl;
#pragma unroll
        for (int st = 0; st < F::kSets; ++st) {
          if constexpr (kWords == 4) {
            uint4 x = *reinterpret_cast<const uint4*>(vp + st * F::kSetDims);
            vw[t][st][0] = x.x; vw[t][st][1] = x.y; vw[t][st][2] = x.z; vw[t][st][3] = x.w;
          } else {
            uint2 x = *reinterpret_cast<const uint2*>(vp + st * F::kSetDims);
            vw[t][st][0] = x.x; vw[t][st][1] = x.y;
          }
        }
      }
#pragma unroll
      for (int st = 0; st < F::kSets; ++st) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
#pragma unroll
          for (int hi = 0; hi < 2; ++hi) {
            // operand for dim st*kSetDims + r16*kDpl + 2w + hi: keys 0..3 of the lane group
            const uint32_t k01 = pack_halves(vw[0][st][w], vw[1][st][w], hi);
            const uint32_t k23 = pack_halves(vw[2][st][w], vw[3][st][w], hi);
            const s16x4_t vop = __builtin_bit_cast(s16x4_t, make_uint2(k01, k23));
            const int blk = st * F::kDpl + 2 * w + hi;
#pragma unroll
            for (int rb = 0; rb < NR; ++rb)
              o[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop[rb], o[rb][blk], 0,
                                                                     0, 0);
          }
        }
      }
    } else {
      // four MFMAs of 4 keys each: step u contracts keys t0 + 4*grp' + u over the lane groups
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = min(t0 + 4 * grp + u, last);
        const float* vp =
            static_cast<const float*>(a.v) + kv_head_off + (size_t)key * D + r16 * 4;
#pragma unroll
        for (int st = 0; st < F::kSets; ++st) {
          const float4 x = *reinterpret_cast<const float4*>(vp + st * F::kSetDims);
          const float xe[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int blk = st * 4 + e;
#pragma unroll
            for (int rb = 0; rb < NR; ++rb)
              o[rb][blk] =
                  __builtin_amdgcn_mfma_f32_16x16x4f32(xe[e], p[rb][u], o[rb][blk], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---------------- partial result of this key range
  const size_t part = (size_t)bhc * n_splits + split;
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const float l_row = xgroup_sum(l_run[rb]);
    if (!row_ok[rb]) continue;
    const int rloc = rb * 16 + r16;
    float* dst = a.ws_o + (part * (16 * NR) + rloc) * D;
    // lane (r16, grp) holds O^T rows 4*grp + j of every 16-dim block:
    //   dim = st*kSetDims + kDpl*(4*grp + j) + u   for block st*kDpl + u
#pragma unroll
    for (int st = 0; st < F::kSets; ++st) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* d0 = dst + st * F::kSetDims + F::kDpl * (4 * grp + j);
#pragma unroll
        for (int u = 0; u < F::kDpl; u += 4) {
          float4 val = make_float4(o[rb][st * F::kDpl + u][j], o[rb][st * F::kDpl + u + 1][j],
                                   o[rb][st * F::kDpl + u + 2][j], o[rb][st * F::kDpl + u + 3][j]);
          *reinterpret_cast<float4*>(d0 + u) = val;
        }
      }
    }
    if (grp == 0) {
      float2 ml = make_float2(m_run[rb], l_row);
      *reinterpret_cast<float2*>(a.ws_ml + (part * (16 * NR) + rloc) * 2) = ml;
    }
  }
}

// One workgroup of 256 threads per output row (b, j, hq). Threads split the row into float4
// columns and the splits into interleaved subsets, then combine through LDS.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int n_splits, int n_chunks,
                                                    int chunk_rows, int nr) {
  constexpr int kCols = D / 4;            // float4 columns of a row
  constexpr int kLanesPerSplit = kCols;   // threads sharing one split
  constexpr int kSplitLanes = 256 / kCols;
  __shared__ float red_m[256];
  __shared__ float4 red_o[256];
  __shared__ float red_l[256];

  const int row_id = blockIdx.x;  // ((b * m + j) * Hq + hq)
  const int hq = row_id % a.n_q_heads;
  const int bj = row_id / a.n_q_heads;
  const int j = bj % a.m;
  const int b = bj / a.m;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int h = hq / G;
  const int row = j * G + (hq % G);
  const int chunk = row / chunk_rows;
  const int rloc = row % chunk_rows;
  const size_t bhc = (size_t)(b * a.n_kv_heads + h) * n_chunks + chunk;
  const size_t base = bhc * n_splits;
  const int rows16 = 16 * nr;

  // pass 1: maximum of the running maxima of non-empty splits
  float M = -INFINITY;
  for (int s = threadIdx.x; s < n_splits; s += 256) {
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + ((base + s) * rows16 + rloc) * 2);
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  red_m[threadIdx.x] = M;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red_m[threadIdx.x] = fmaxf(red_m[threadIdx.x], red_m[threadIdx.x + off]);
    __syncthreads();
  }
  M = red_m[0];

  // pass 2: rescaled sums
  const int col = threadIdx.x % kLanesPerSplit;
  const int sl = threadIdx.x / kLanesPerSplit;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  for (int s = sl; s < n_splits; s += kSplitLanes) {
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + ((base + s) * rows16 + rloc) * 2);
    if (ml.y > 0.f) {
      const float w = __builtin_amdgcn_exp2f(ml.x - M);
      L += w * ml.y;
      const float4 x =
          *reinterpret_cast<const float4*>(a.ws_o + ((base + s) * rows16 + rloc) * D + col * 4);
      acc.x += w * x.x; acc.y += w * x.y; acc.z += w * x.z; acc.w += w * x.w;
    }
  }
  red_o[threadIdx.x] = acc;
  red_l[threadIdx.x] = L;
  __syncthreads();
  for (int off = kSplitLanes / 2; off > 0; off >>= 1) {
    if (sl < off) {
      const int o2 = threadIdx.x + off * kLanesPerSplit;
      float4 x = red_o[o2];
      red_o[threadIdx.x].x += x.x; red_o[threadIdx.x].y += x.y;
      red_o[threadIdx.x].z += x.z; red_o[threadIdx.x].w += x.w;
      red_l[threadIdx.x] += red_l[o2];
    }
    __syncthreads();
  }
  if (sl == 0) {
    const float Lt = red_l[col];
    float4 r = red_o[col];
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    if (Lt > 0.f) {
      const float inv = 1.f / Lt;
      res = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    }
    *reinterpret_cast<float4*>(a.out + (size_t)row_id * D + col * 4) = res;
    if (col == 0 && a.lse) a.lse[row_id] = (Lt > 0.f) ? (M + log2f(Lt)) * kLn2 : -INFINITY;
  }
}

template <int D, bool BF16>
hipError_t launch_split(const AttnArgs& a, const SplitPlan& p, hipStream_t stream) {
  dim3 grid((p.n_splits + kWavesPerBlock - 1) / kWavesPerBlock,
            a.batch * a.n_kv_heads * p.n_chunks);
  dim3 block(64 * kWavesPerBlock);
  // row blocks beyond the register budget of (D, dtype) are never planned (rows_cap)
  constexpr int kMaxNr = BF16 ? (D == 256 ? 2 : 4) : (D == 64 ? 4 : (D == 128 ? 2 : 1));
  if (p.nr < 1 || p.nr > kMaxNr) return hipErrorInvalidValue;
  switch (p.nr) {
    case 1: attn_split_kernel<D, 1, BF16><<<grid, block, 0, stream>>>(a, p.n_splits, p.keys_per_split, p.n_chunks, p.chunk_rows); break;
    case 2: if constexpr (kMaxNr >= 2) attn_split_kernel<D, 2, BF16><<<grid, block, 0, stream>>>(a, p.n_splits, p.keys_per_split, p.n_chunks, p.chunk_rows); break;
    case 3: if constexpr (kMaxNr >= 3) attn_split_kernel<D, 3, BF16><<<grid, block, 0, stream>>>(a, p.n_splits, p.keys_per_split, p.n_chunks, p.chunk_rows); break;
    default: if constexpr (kMaxNr >= 4) attn_split_kernel<D, 4, BF16><<<grid, block, 0, stream>>>(a, p.n_splits, p.keys_per_split, p.n_chunks, p.chunk_rows); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  merge_kernel<D><<<dim3(a.batch * a.m * a.n_q_heads), dim3(256), 0, stream>>>(
      a, p.n_splits, p.n_chunks, p.chunk_rows, p.nr);
  return hipGetLastError();
}

}  // namespace

// Largest row chunk whose Q operand and O accumulators fit the register file beside the K/V tiles.
static int rows_cap(int dtype, int head_dim) {
  if (dtype == WMTP_BF16) return head_dim == 256 ? 32 : 64;
  return head_dim == 64 ? 64 : (head_dim == 128 ? 32 : 16);
}

bool make_plan_for(int batch, int n_q_heads, int n_kv_heads, int head_dim, int m,
                            int max_seq_len, int dtype, SplitPlan* p) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads) return false;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return false;
  if (m < 1 || m > kMaxM || max_seq_len < 1) return false;
  p->G = n_q_heads / n_kv_heads;
  p->rows = p->G * m;
  const int cap = rows_cap(dtype, head_dim);
  p->chunk_rows = p->rows < cap ? p->rows : cap;
  p->n_chunks = (p->rows + p->chunk_rows - 1) / p->chunk_rows;
  p->nr = (p->chunk_rows + 15) / 16;
  const long long bhc = (long long)batch * n_kv_heads * p->n_chunks;
  const long long tiles_per_seq = ((long long)max_seq_len + kTileKeys - 1) / kTileKeys;
  long long tps = (bhc * tiles_per_seq + kTargetWaves - 1) / kTargetWaves;
  if (tps < 1) tps = 1;
  if (tps > tiles_per_seq) tps = tiles_per_seq;
  p->keys_per_split = (int)(tps * kTileKeys);
  p->n_splits = (int)((max_seq_len + (long long)p->keys_per_split - 1) / p->keys_per_split);
  p->ws_o_floats = (size_t)bhc * p->n_splits * 16 * p->nr * head_dim;
  p->ws_ml_floats = (size_t)bhc * p->n_splits * 16 * p->nr * 2;
  return true;
}

hipError_t launch_attention(const AttnArgs& a, const SplitPlan& p, int dtype, hipStream_t stream) {
  const bool bf16 = dtype == WMTP_BF16;
  switch (a.head_dim) {
    case 64: return bf16 ? launch_split<64, true>(a, p, stream) : launch_split<64, false>(a, p, stream);
    case 128: return bf16 ? launch_split<128, true>(a, p, stream) : launch_split<128, false>(a, p, stream);
    case 256: return bf16 ? launch_split<256, true>(a, p, stream) : launch_split<256, false>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp
