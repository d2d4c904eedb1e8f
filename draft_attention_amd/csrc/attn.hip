// attn.hip -- split-K flash-decoding attention for gfx950 (MI355X), used by the attention entry
// points: the Windowed-MTP draft step (attend the sinks and recent window held by a ring buffer),
// the native full-context draft step and the target's causal verification of m draft candidates
// (Windowed-MTP abstract, third and fifth sentences: the native draft attends the whole KV cache;
// the windowed draft attends sinks plus a recent window; verification stays full attention), and
// the MASW-style step (two reads merged into one result).
//
// Kernel 1 (attn_split_kernel, up to 16*NR query rows per KV head): one workgroup of four 64-lane
// wavefronts owns a share of the keys of one (sequence, KV head, row chunk). The G*m query rows of
// a KV head form one dense operand (GQA), so both products run on the matrix cores:
//   S^T (16 keys x 16 rows) = K_tile (16 x d) . Q^T          v_mfma_f32_16x16x32_bf16 / 16x16x4_f32
//   O^T (16 dims x 16 rows) += V_tile^T (16 x 16 keys) . P^T  v_mfma_f32_16x16x16_bf16 / 16x16x4_f32
// With this orientation every lane of both results holds one query row (lane & 15), so the
// running max, running sum and the rescaling of O are per-lane scalars, and the softmax weights
// left in the S^T registers are already the P^T operand of the second product: the inner loop uses
// no LDS, and cross-lane traffic only on the rare tiles that move a row's reference maximum.
// K rows are read straight from HBM into the operand layout (16-byte loads, 64 contiguous bytes per
// key per instruction). V rows are read with each 16-lane group streaming one key's row and are
// transposed in registers with v_perm_b32 into the V^T operand. 16-key tiles are dealt grid-stride
// over all wavefronts of the launch (all workgroups sweep the cache together), and each wavefront
// keeps the next tile's loads in flight while it computes the current one. At the end the
// wavefronts combine their states through LDS, each wavefront a quarter of the dims, into one
// partial (o unnormalised, running max in log2 units, running sum) per query row.
//
// Kernel 1 also takes a verification of up to three row blocks (48 rows) when they fit one row
// chunk. Kernel 1b (attn_coop_kernel, more rows: verification): the wavefronts of a workgroup
// (four, or eight for eight row blocks) share each tile through an LDS stage (see the comment
// above the kernel).
//
// Kernel 2 (merge_kernel): log-sum-exp merge of the partials of every output row, one workgroup per
// (row, 32 or 64 dims):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s o_s 2^(m_s - M) / L,  lse = (M + log2 L) ln 2.

#include <algorithm>
#include <type_traits>

#include "wmtp_internal.h"

namespace wmtp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// K and V are streamed once per call: nontemporal loads keep them from displacing useful lines in
// the caches (measured on MI355X: the full 1M-token read goes from 6.0 to 6.7 TB/s).
__device__ __forceinline__ uint4 stream_load16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ uint2 stream_load8(const void* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(static_cast<const u32x2_t*>(p)));
}

// Requests every kernel argument in one round of scalar loads. Left alone, the compiler loads the
// fields in the order the code first needs them, waiting between rounds: two or three dependent
// round trips to the kernel-argument segment before the first vector load. Used by the merge
// (a few microseconds in all) and the cooperative kernel; measured on MI355X, the split kernel
// (whose first rounds overlap its integer set-up) is as fast or faster without it.
__device__ __forceinline__ void request_args(const AttnArgs& a) {
  asm volatile("" ::"s"(a.q), "s"(a.k), "s"(a.v), "s"(a.seq_len), "s"(a.out), "s"(a.lse),
               "s"(a.ws_o), "s"(a.ws_ml), "s"(a.batch), "s"(a.n_kv_heads), "s"(a.n_q_heads),
               "s"(a.m), "s"(a.capacity), "s"(a.limit), "s"(a.mode), "s"(a.sm_scale), "s"(a.sink),
               "s"(a.window), "s"(a.wphys), "s"(a.part_stride), "s"(a.part_offset), "s"(a.new_k),
               "s"(a.new_v), "s"(a.pos));
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ unsigned div_of(unsigned x, const FastDiv& f) {
  return (__umulhi(x, f.mul) + x) >> f.shift;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.f;  // softmax weights stay below 2^8 between rescales
constexpr int kThreads = 64 * kWavesPerBlock;

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

// Two bf16 from the low (hi = false) or high halves of two dwords, a's half in the low 16 bits.
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, bool hi) {
  return __builtin_amdgcn_perm(b, a, hi ? 0x07060302u : 0x05040100u);
}

template <int D, bool BF16>
struct Frag {
  static constexpr int kEB = BF16 ? 2 : 4;                // bytes per element
  static constexpr int kQRegs = BF16 ? D / 32 : D / 16;    // 16-byte K/Q pieces per lane per key
  static constexpr int kDpl = BF16 ? (D >= 128 ? 8 : 4) : 4;  // V dims per lane per set
  static constexpr int kSetDims = 16 * kDpl;
  static constexpr int kSets = D / kSetDims;
  static constexpr int kBlocks = D / 16;                   // 16-dim output blocks
  static constexpr int kVWords = BF16 ? kDpl / 2 : 4;      // dwords per (key, set)
};

// One 16-key tile in registers: the K operand of S^T and four keys' worth of V per lane.
template <int D, bool BF16>
struct Tile {
  using F = Frag<D, BF16>;
  uint4 k[F::kQRegs];
  uint32_t v[4][F::kSets][F::kVWords];
};

// Keys t0..t0+15 (indices past `last` read row `last`; their scores are masked).
// The slot `fresh` (-1: none) is read from the rows knew/vnew instead of the cache: the token a
// fused draft step appends, whose slot is written in the same launch.
template <int D, bool BF16>
__device__ __forceinline__ void load_tile(const char* kbase, const char* vbase, int t0, int last,
                                          int r16, int grp, Tile<D, BF16>& T, int fresh = -1,
                                          const char* knew = nullptr, const char* vnew = nullptr) {
  using F = Frag<D, BF16>;
  const int key = min(t0 + r16, last);
  const char* krow = key == fresh ? knew : kbase + (size_t)key * D * F::kEB;
  const uint4* kp = reinterpret_cast<const uint4*>(krow);
#pragma unroll
  for (int ks = 0; ks < F::kQRegs; ++ks) T.k[ks] = stream_load16(kp + ks * 4 + grp);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kv = min(t0 + 4 * grp + t, last);
    const char* vrow = kv == fresh ? vnew : vbase + (size_t)kv * D * F::kEB;
    const char* vp = vrow + (size_t)r16 * F::kDpl * F::kEB;
#pragma unroll
    for (int st = 0; st < F::kSets; ++st) {
      if constexpr (F::kVWords == 4) {
        const uint4 x = stream_load16(vp + st * F::kSetDims * F::kEB);
        T.v[t][st][0] = x.x; T.v[t][st][1] = x.y; T.v[t][st][2] = x.z; T.v[t][st][3] = x.w;
      } else {
        const uint2 x = stream_load8(vp + st * F::kSetDims * F::kEB);
        T.v[t][st][0] = x.x; T.v[t][st][1] = x.y;
      }
    }
  }
}

// The query operand of S^T = K . Q^T for this lane: fragment (rb, ks) holds row rb*16 + (lane & 15),
// dims ks*32 + (lane >> 4)*8 .. +7 (bf16) or ks*16 + (lane >> 4)*4 .. +3 (fp32). It lives either in
// registers or in LDS (read back once per tile; consecutive lanes read consecutive 16 bytes, so the
// reads are conflict-free): in LDS when it would crowd out the K/V tiles, or when FORCE_LDS asks
// for one load per workgroup instead of one per wavefront (short reads, see the planner).
template <int D, int NR, bool BF16, bool FORCE_LDS = false>
struct QOperand {
  using F = Frag<D, BF16>;
  typedef typename std::conditional<BF16, bf16x8_t, f32x4_t>::type Vec;
  static constexpr bool kInLds = FORCE_LDS || NR * F::kQRegs * 4 >= 64;
  Vec reg[kInLds ? 1 : NR][kInLds ? 1 : F::kQRegs];
  const uint4* lds;
  int lane;
  __device__ __forceinline__ Vec get(int rb, int ks) const {
    if constexpr (kInLds)
      return __builtin_bit_cast(Vec, lds[(rb * F::kQRegs + ks) * 64 + lane]);
    else
      return reg[rb][ks];
  }
};

template <int D, int NR, bool BF16>
struct RowState {
  float m[NR];  // reference max (log2 units, within 2^8 of the running max), same on a row's lanes
  float l[NR];  // this lane's share of the running sum
  f32x4_t o[NR][Frag<D, BF16>::kBlocks];
};

// Windowed read of a ring with slack (capacity = S + W + slack): every slot is scanned and a slot
// is attended iff it holds a sink (slot s < min(S, n)) or one of the last W positions. The window
// slots hold positions in wrap order, so the age of window slot S + u (0 = newest position) is
// (top - u) mod Wp with top = (n - 1 - S) mod Wp, Wp = W + slack, and the slot is attended iff its
// age < min(W, n - S). The test depends on n alone, so loads never wait for it.
struct RingMask {
  bool active;
  int n, sink, wphys, top, wcount;
  __device__ __forceinline__ bool attended(int s) const {
    if (s < sink) return s < n;
    int age = top - (s - sink);
    age += age < 0 ? wphys : 0;
    return age < wcount;
  }
};

// A windowed read of a ring with slack slots (kernels instantiated with RING = true).
inline bool ring_masked(const AttnArgs& a) { return a.mode == kModeWindowed && a.wphys > a.window; }

__device__ __forceinline__ RingMask ring_mask(const AttnArgs& a, int raw_n) {
  RingMask r;
  r.active = a.mode == kModeWindowed && a.wphys > a.window;
  r.n = raw_n;
  r.sink = a.sink;
  r.wphys = a.wphys > 0 ? a.wphys : 1;
  r.top = 0;
  r.wcount = 0;
  if (r.active && raw_n > a.sink) {  // the modulo only for rings with slack
    r.top = (raw_n - 1 - a.sink) % r.wphys;
    r.wcount = min(a.window, raw_n - a.sink);
  }
  return r;
}

// S^T = K_tile . Q^T of one tile (the score products; they do not depend on the running state)
template <int D, int NR, bool BF16, typename QOp>
__device__ __forceinline__ void tile_scores(const Tile<D, BF16>& T, const QOp& qf, f32x4_t (&s)[NR]) {
  using F = Frag<D, BF16>;
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) s[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (BF16) {
#pragma unroll
    for (int ks = 0; ks < F::kQRegs; ++ks)
#pragma unroll
      for (int rb = 0; rb < NR; ++rb)
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, T.k[ks]),
                                                        qf.get(rb, ks), s[rb], 0, 0, 0);
  } else {
#pragma unroll
    for (int ks = 0; ks < F::kQRegs; ++ks) {
      const float4 kf = __builtin_bit_cast(float4, T.k[ks]);
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        const f32x4_t q4 = qf.get(rb, ks);
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x, q4[0], s[rb], 0, 0, 0);
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.y, q4[1], s[rb], 0, 0, 0);
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.z, q4[2], s[rb], 0, 0, 0);
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.w, q4[3], s[rb], 0, 0, 0);
      }
    }
  }
}

// The online-softmax update of the running state with one tile whose scores s are given.
template <int D, int NR, bool BF16, bool RING>
__device__ __forceinline__ void tile_update(const Tile<D, BF16>& T, const f32x4_t (&s)[NR], int t0,
                                            int last, const int (&last_visible)[NR],
                                            const RingMask& rm, int grp, float scale_log2,
                                            RowState<D, NR, BF16>& st) {
  using F = Frag<D, BF16>;
  // ---------------- online softmax; this lane holds keys t0 + 4*grp + j (j = 0..3) of its row.
  // The weights are taken relative to a reference maximum st.m that only moves when a tile's
  // maximum exceeds it by more than kRescaleLog2 (softmax does not depend on the reference), so
  // the weights stay below 2^kRescaleLog2 and the O accumulators are rescaled only on the rare
  // tiles where some row's reference moves (a wavefront-uniform branch). Each lane first tests
  // its own four keys; only when one of them passes the threshold does the wavefront take the
  // row maximum over the row's four lanes (no cross-lane traffic on the common path; the outcome
  // is the same as testing the row maximum on every tile).
  float sc[NR][4];
  bool need = false;
  float mx[NR];
  bool ring_ok[4] = {true, true, true, true};
  if constexpr (RING) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ring_ok[j] = rm.attended(t0 + 4 * grp + j);
  }
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int vis = min(last, last_visible[rb]);
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = t0 + 4 * grp + j;
      sc[rb][j] = (key <= vis && ring_ok[j]) ? s[rb][j] * scale_log2 : -INFINITY;
      m = fmaxf(m, sc[rb][j]);
    }
    mx[rb] = m;
    need |= m > st.m[rb] + kRescaleLog2;
  }
  if (__ballot(need)) {
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
      mx[rb] = xgroup_max(mx[rb]);
      // rows whose reference stays put keep alpha = 1 exactly (their st.m may still be -inf
      // when the causal mask hid every key so far, and -inf - -inf is not a number)
      const bool moved = mx[rb] > st.m[rb] + kRescaleLog2;
      const float alpha = moved ? __builtin_amdgcn_exp2f(st.m[rb] - mx[rb]) : 1.f;  // 0 from -inf
      st.l[rb] *= alpha;
#pragma unroll
      for (int i = 0; i < F::kBlocks; ++i) st.o[rb][i] *= alpha;
      st.m[rb] = moved ? mx[rb] : st.m[rb];
    }
  }
  float p[NR][4];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const float m_use = (st.m[rb] == -INFINITY) ? 0.f : st.m[rb];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[rb][j] = __builtin_amdgcn_exp2f(sc[rb][j] - m_use);
      psum += p[rb][j];
    }
    st.l[rb] += psum;
  }

  // ---------------- O^T += V_tile^T . P^T
  if constexpr (BF16) {
    s16x4_t pop[NR];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
      const bf16x4_t pb =
          __builtin_convertvector(f32x4_t{p[rb][0], p[rb][1], p[rb][2], p[rb][3]}, bf16x4_t);
      pop[rb] = __builtin_bit_cast(s16x4_t, pb);
    }
#pragma unroll
    for (int sx = 0; sx < F::kSets; ++sx) {
#pragma unroll
      for (int w = 0; w < F::kVWords; ++w) {
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          // dim sx*kSetDims + r16*kDpl + 2w + hi of keys 4*grp + 0..3
          const uint32_t k01 = pack_halves(T.v[0][sx][w], T.v[1][sx][w], hi);
          const uint32_t k23 = pack_halves(T.v[2][sx][w], T.v[3][sx][w], hi);
          const s16x4_t vop = __builtin_bit_cast(s16x4_t, make_uint2(k01, k23));
          const int blk = sx * F::kDpl + 2 * w + hi;
#pragma unroll
          for (int rb = 0; rb < NR; ++rb)
            st.o[rb][blk] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop[rb], st.o[rb][blk], 0, 0, 0);
        }
      }
    }
  } else {
    // four MFMAs of 4 keys: step u contracts keys 4*grp' + u over the lane groups grp'
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int sx = 0; sx < F::kSets; ++sx) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ve = __builtin_bit_cast(float, T.v[u][sx][e]);
          const int blk = sx * 4 + e;
#pragma unroll
          for (int rb = 0; rb < NR; ++rb)
            st.o[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(ve, p[rb][u], st.o[rb][blk], 0,
                                                                 0, 0);
        }
      }
    }
  }
}

template <int D, int NR, bool BF16, bool RING, typename QOp>
__device__ __forceinline__ void compute_tile(const Tile<D, BF16>& T, const QOp& qf, int t0,
                                             int last, const int (&last_visible)[NR],
                                             const RingMask& rm, int grp, float scale_log2,
                                             RowState<D, NR, BF16>& st) {
  f32x4_t s[NR];
  tile_scores<D, NR, BF16>(T, qf, s);
  tile_update<D, NR, BF16, RING>(T, s, t0, last, last_visible, rm, grp, scale_log2, st);
}

// Lane (r16, grp) holds O^T rows 4*grp + j of every 16-dim block; block sx*kDpl + u covers
// dims sx*kSetDims + kDpl*(4*grp + j) + u. These are four runs of kDpl contiguous dims per set.
template <int D, bool BF16>
__device__ __forceinline__ int out_dim(int sx, int grp, int j) {
  using F = Frag<D, BF16>;
  return sx * F::kSetDims + F::kDpl * (4 * grp + j);
}

// Zeroes the V rows of the tile's keys past `last`. Their weights are 0, but 0 * NaN is NaN: the
// first tile of a wavefront is requested against the host-side bound before seq_len is known, so
// its keys past the length hold whatever those rows hold. Called on a wavefront-uniform branch,
// only for a tile that reaches past `last`.
template <int D, bool BF16>
__device__ __forceinline__ void clear_past(Tile<D, BF16>& T, int t0, int last, int grp) {
  using F = Frag<D, BF16>;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool keep = t0 + 4 * grp + j <= last;
#pragma unroll
    for (int sx = 0; sx < F::kSets; ++sx)
#pragma unroll
      for (int w = 0; w < F::kVWords; ++w) T.v[j][sx][w] = keep ? T.v[j][sx][w] : 0u;
  }
}

// Whether a wavefront can hold two tiles (the next one in flight) beside its query operand and
// accumulators without spilling: a register estimate in 32-bit registers per lane.
template <int D, int NR, bool BF16>
constexpr bool pipelined() {
  using F = Frag<D, BF16>;
  constexpr int q = QOperand<D, NR, BF16>::kInLds ? 0 : NR * F::kQRegs * 4;
  constexpr int o = NR * F::kBlocks * 4;
  constexpr int tile = F::kQRegs * 4 + 4 * F::kSets * F::kVWords;
  return q + o + 2 * tile <= 224 && o <= 96;
}

// QLDS: the query operand is loaded once per workgroup and read from LDS (short reads).
template <int D, int NR, bool BF16, bool RING, bool FUSED, bool QLDS>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnArgs a, int n_splits,
                                                              int n_chunks, int chunk_rows) {
  using F = Frag<D, BF16>;
  constexpr int kRows = 16 * NR;
  constexpr int kPitch = D + 4;  // LDS row pitch (floats): rows start 4 banks apart
  __shared__ float sm_o[kWavesPerBlock][kRows * kPitch];
  __shared__ float2 sm_ml[kWavesPerBlock][kRows];

  const int lane = threadIdx.x & 63;
  // the wavefront index is uniform across the wavefront: in a scalar register, tile indices and
  // loop conditions derived from it stay scalar (uniform branches instead of exec-mask loops,
  // whose merged paths made the compiler wait for most of a tile before requesting the next)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x;
  const int bhc = blockIdx.y;
  // (divisions by the call's invariant sizes as multiply-shifts: every operand is below 2^31)
  const int bh = div_of(bhc, a.div_chunks);
  const int chunk = bhc - bh * n_chunks;
  const int b = div_of(bh, a.div_kv);
  const int h = bh - b * a.n_kv_heads;
  const int G = a.div_g.d;
  const int rows = G * a.m;
  const int row0 = chunk * chunk_rows;
  const int row_end = min(rows, row0 + chunk_rows);

  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const size_t head_off = (size_t)(b * a.n_kv_heads + h) * (size_t)a.capacity * D * F::kEB;
  const char* kbase = static_cast<const char*>(a.k) + head_off;
  const char* vbase = static_cast<const char*>(a.v) + head_off;

  // ---- query rows of this lane: row = row0 + rb*16 + r16 -> candidate jq, head hq. The query
  // loads go out first, ahead of the first tile: every later wait for a tile then also covers
  // them, on the first pass through the tile loop as on the others.
  using QOp = QOperand<D, NR, BF16, QLDS>;
  static_assert(!QOp::kInLds || NR <= kWavesPerBlock, "one row block per wavefront for the LDS copy");
  __shared__ uint4 sm_q[QOp::kInLds ? NR * F::kQRegs * 64 : 1];
  int row_j[NR];  // candidate index of the row
  bool row_ok[NR];
  QOp qf;
  qf.lds = sm_q;
  qf.lane = lane;
  uint4 qraw[QOp::kInLds ? F::kQRegs : 1];  // LDS copy: this wavefront's row block, stored later
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int row = row0 + rb * 16 + r16;
    row_ok[rb] = row < row_end;
    // padding rows load the last real row (never written out; no select, so no early wait)
    const int row_q = row_ok[rb] ? row : row_end - 1;
    const int jq = div_of(row_q, a.div_g);
    const int hq = h * G + (row_q - jq * G);
    row_j[rb] = jq;
    if (QOp::kInLds && rb != wave) continue;  // LDS copy: one wave per row block
    const size_t qoff = ((size_t)(b * a.m + jq) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int ks = 0; ks < F::kQRegs; ++ks) {
      // bf16: dims ks*32 + grp*8 .. +7; fp32: dims ks*16 + grp*4 .. +3 (the chunk K holds)
      const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                        qoff * F::kEB + (ks * 4 + grp) * 16);
      if constexpr (QOp::kInLds)
        qraw[ks] = raw;
      else
        qf.reg[rb][ks] = __builtin_bit_cast(typename QOp::Vec, raw);
    }
  }

  // Tiles are dealt grid-stride: wavefront (split, wave) takes tiles (split*4 + wave) + k*(4*
  // n_splits), so all workgroups sweep the cache together (the access pattern HBM streams best);
  // the log-sum-exp merge does not care which keys a partial holds. Loads are clamped to row
  // `last` and issued unconditionally (a prefetch past the end re-reads row `last` and is never
  // used), so the compiler waits for exactly the older tile instead of draining every outstanding
  // load. capacity <= 2^30 and kStride <= 64 * (the planner's workgroup target, 256) keep every
  // index, t + 2 * kStride included, below 2^31.
  const int kStride = n_splits * kWavesPerBlock * kTileKeys;
  int t = (split * kWavesPerBlock + wave) * kTileKeys;
  Tile<D, BF16> A, B;
  // The first tile is requested against the host-side bound (a.limit >= 1, so row limit-1 is
  // always a valid address) without waiting for seq_len: the loads overlap the seq_len read, and
  // seq_len only masks. Later tiles clamp to the last real key. (A wavefront without tiles reads
  // row limit-1; the request is unconditional so that every path into the tile loop has the same
  // loads outstanding.)
  load_tile<D, BF16>(kbase, vbase, t, min(a.limit - 1, t + kTileKeys - 1), r16, grp, A);

  int n = a.seq_len[b];
  n = max(n, 0);
  // fused draft step: the token at position n (its slot `fresh`) joins the attended set
  int fresh = -1;
  const char* knew = nullptr;
  const char* vnew = nullptr;
  if constexpr (FUSED) {
    const int64_t p = n;
    const int64_t slot = a.wphys == 0 ? p : (p < a.sink ? p : a.sink + (p - a.sink) % a.wphys);
    const size_t new_off = (size_t)(b * a.n_kv_heads + h) * D * F::kEB;
    knew = static_cast<const char*>(a.new_k) + new_off;
    vnew = static_cast<const char*>(a.new_v) + new_off;
    if (slot < a.capacity) {
      fresh = (int)slot;
      if (split == 0 && chunk == 0) {  // one workgroup per KV head stores the token
        constexpr int kPieces = D * F::kEB / 16;
        for (int i = threadIdx.x; i < 2 * kPieces; i += kThreads) {
          if (i < kPieces)
            reinterpret_cast<uint4*>(const_cast<char*>(kbase) + (size_t)slot * D * F::kEB)[i] =
                reinterpret_cast<const uint4*>(knew)[i];
          else
            reinterpret_cast<uint4*>(const_cast<char*>(vbase) + (size_t)slot * D * F::kEB)[i - kPieces] =
                reinterpret_cast<const uint4*>(vnew)[i - kPieces];
        }
        if (h == 0 && threadIdx.x == 0 && a.pos) a.pos[(size_t)b * a.capacity + slot] = (int32_t)p;
      }
    }
    n = n < 0x7fffffff ? n + 1 : n;
    // the first tile went out before `fresh` was known: the one wavefront whose first tile holds
    // the new token's slot fetches that tile again, reading the token from knew/vnew
    if (t < a.limit && fresh >= t && fresh < t + kTileKeys)
      load_tile<D, BF16>(kbase, vbase, t, min(a.limit - 1, t + kTileKeys - 1), r16, grp, A, fresh,
                         knew, vnew);
  }
  const RingMask rm = ring_mask(a, n);
  n = min(n, a.limit);
  const int last = n - 1;

  int last_visible[NR];  // largest key index the row may attend
#pragma unroll
  for (int rb = 0; rb < NR; ++rb)
    last_visible[rb] = (a.mode == kModeVerify) ? (n - a.m + row_j[rb]) : (n - 1);
  if constexpr (QOp::kInLds) {
    if (wave < NR) {
#pragma unroll
      for (int ks = 0; ks < F::kQRegs; ++ks) sm_q[(wave * F::kQRegs + ks) * 64 + lane] = qraw[ks];
    }
    __syncthreads();
  }

  const float scale_log2 = a.sm_scale * kLog2e;
  RowState<D, NR, BF16> st;
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int i = 0; i < F::kBlocks; ++i) st.o[rb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if constexpr (pipelined<D, NR, BF16>()) {
    // software-pipelined tile loop: two register tiles, the next one always in flight. A round
    // takes two tiles and has no exit in its middle: the second tile's successor is requested
    // (clamped) even when the second tile is past the end and is not computed. Every path then
    // reaches each tile's first use with the same loads issued after it, so the compiler waits for
    // exactly that tile (an exit inside the round, or a conditional request, made it wait for most
    // of a tile before requesting the next). The scheduling barriers keep each request ahead of
    // the computation it overlaps.
    if (t < n && t + kStride >= n) {
      // a single tile (the windowed read's usual share): nothing to overlap
      if (t + kTileKeys - 1 > last) clear_past<D, BF16>(A, t, last, grp);
      compute_tile<D, NR, BF16, RING>(A, qf, t, last, last_visible, rm, grp, scale_log2, st);
      t = n;
    }
    while (t < n) {
      load_tile<D, BF16>(kbase, vbase, t + kStride, last, r16, grp, B, fresh, knew, vnew);
      __builtin_amdgcn_sched_barrier(0);
      if (t + kTileKeys - 1 > last) clear_past<D, BF16>(A, t, last, grp);
      compute_tile<D, NR, BF16, RING>(A, qf, t, last, last_visible, rm, grp, scale_log2, st);
      load_tile<D, BF16>(kbase, vbase, t + 2 * kStride, last, r16, grp, A, fresh, knew, vnew);
      __builtin_amdgcn_sched_barrier(0);
      if (t + kStride < n) {
        if (t + kStride + kTileKeys - 1 > last) clear_past<D, BF16>(B, t + kStride, last, grp);
        compute_tile<D, NR, BF16, RING>(B, qf, t + kStride, last, last_visible, rm, grp, scale_log2,
                                        st);
      }
      t += 2 * kStride;
    }
  } else {
    // one register tile: loads of tile t + stride start once tile t is consumed
    (void)B;
    while (t < n) {
      if (t + kTileKeys - 1 > last) clear_past<D, BF16>(A, t, last, grp);
      compute_tile<D, NR, BF16, RING>(A, qf, t, last, last_visible, rm, grp, scale_log2, st);
      t += kStride;
      if (t < n) load_tile<D, BF16>(kbase, vbase, t, last, r16, grp, A, fresh, knew, vnew);
    }
  }

  float l_row[NR];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) l_row[rb] = xgroup_sum(st.l[rb]);

  // ---- combine the four wavefronts' states through LDS: every wavefront stores its state, then
  // wavefront w combines dims [w*D/4, (w+1)*D/4) of every row of the workgroup and writes that
  // part of the partial (the four share the combining work and the stores)
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
    const int rloc = rb * 16 + r16;
    float* dst = &sm_o[wave][rloc * kPitch];
#pragma unroll
    for (int sx = 0; sx < F::kSets; ++sx)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int u = 0; u < F::kDpl; u += 4)
          *reinterpret_cast<float4*>(dst + out_dim<D, BF16>(sx, grp, j) + u) =
              make_float4(st.o[rb][sx * F::kDpl + u][j], st.o[rb][sx * F::kDpl + u + 1][j],
                          st.o[rb][sx * F::kDpl + u + 2][j], st.o[rb][sx * F::kDpl + u + 3][j]);
    if (grp == 0) sm_ml[wave][rloc] = make_float2(st.m[rb], l_row[rb]);
  }
  __syncthreads();

  const size_t part = (size_t)bhc * a.part_stride + a.part_offset + split;
  constexpr int kQuarter = D / kWavesPerBlock;  // dims combined by one wavefront
  constexpr int kF4 = kQuarter / 4;             // their float4 columns per row
  static_assert((16 * kF4) % 64 == 0, "a row block's quarter spreads evenly over the lanes");
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
    for (int it = 0; it < 16 * kF4 / 64; ++it) {
      const int item = lane + 64 * it;
      const int rloc = rb * 16 + item / kF4;
      const int dim = wave * kQuarter + 4 * (item % kF4);
      float mw[kWavesPerBlock], lw[kWavesPerBlock];
      float M = -INFINITY;
#pragma unroll
      for (int x = 0; x < kWavesPerBlock; ++x) {
        const float2 ml = sm_ml[x][rloc];
        mw[x] = ml.x;
        lw[x] = ml.y;
        M = fmaxf(M, ml.x);
      }
      const float m_use = (M == -INFINITY) ? 0.f : M;
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int x = 0; x < kWavesPerBlock; ++x) {
        const float wgt = __builtin_amdgcn_exp2f(mw[x] - m_use);
        L += wgt * lw[x];
        const float4 y = *reinterpret_cast<const float4*>(&sm_o[x][rloc * kPitch + dim]);
        acc.x += wgt * y.x; acc.y += wgt * y.y;
        acc.z += wgt * y.z; acc.w += wgt * y.w;
      }
      if (row0 + rloc >= row_end) continue;  // padding row
      *reinterpret_cast<float4*>(a.ws_o + (part * kRows + rloc) * D + dim) = acc;
      if (wave == 0 && item % kF4 == 0)
        *reinterpret_cast<float2*>(a.ws_ml + (part * kRows + rloc) * 2) = make_float2(M, L);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Cooperative-tile kernel. The wavefronts of a workgroup (four, or eight: Coop::kWaves) consume the
// SAME 16-key tile, which the whole workgroup stages through LDS: every thread issues fully coalesced 16-byte loads for its
// share of the tile (K and V rows are contiguous in HBM), keeps kPrefetch tiles of them in flight
// in registers, and writes the oldest one into a double-buffered LDS stage (K chunks XOR-swizzled
// by key so the operand reads below are bank-conflict free). One barrier per tile.
// The wavefronts split the work of a tile by query-row block (NB = 4: one block of 16 rows each,
// the verify shape; NB = 8: one block each on eight wavefronts, or two blocks each on four,
// sharing one V operand read) or by output dimensions (NB = 1 or 2: each wavefront owns D/4 or D/2
// dims of its block's rows and recomputes the 16x16 score tile, which is cheap on the matrix
// cores). Each wavefront writes its own part of the workgroup's partial; no cross-wavefront merge
// is needed.
#ifndef WMTP_COOP_EIGHT_WAVES
#define WMTP_COOP_EIGHT_WAVES 1
#endif
template <int D, int NB, bool BF16>
struct Coop {
  static constexpr int kEB = BF16 ? 2 : 4;
  static constexpr int kRowBytes = D * kEB;
  static constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per key row
  static constexpr int kSwz = (kChunks < 16 ? kChunks : 16) - 1;
  static constexpr int kVSwz = (kChunks / 2 < 8 ? kChunks / 2 : 8) - 1;  // 32-byte segments of V
  static constexpr int kTileBytes = 16 * kRowBytes;           // K (or V) bytes of one tile
#ifdef WMTP_COOP_TPS
  static constexpr int kTps = WMTP_COOP_TPS;                   // tiles per LDS stage (per barrier)
#else
  static constexpr int kTps = 1;
#endif
  static constexpr int kStageBytes = kTps * 2 * kTileBytes;   // K and V of the stage's tiles
  // Wavefronts per workgroup: eight for eight row blocks (one block each) when a stage gives each
  // of the 512 threads a 16-byte load, else four. Measured on MI355X (verification at L = 1M,
  // 32q/2kv, d128, bf16): eight blocks on eight wavefronts 230 us, on four (two blocks each)
  // 236-241 us; with the padding blocks skipped (below) 80 rows take 185 us instead of 238. Four
  // blocks on eight wavefronts (each half the dims of one block) took 198 us against 174.
  static constexpr int kWaves =
      (WMTP_COOP_EIGHT_WAVES && NB == 8 && kStageBytes >= 16 * 512) ? 8 : kWavesPerBlock;
  static constexpr int kThreadsC = 64 * kWaves;
  static constexpr int kRbw = NB > kWaves ? NB / kWaves : 1;    // row blocks per wavefront
  static constexpr int kSplitD = NB >= kWaves ? 1 : kWaves / NB;  // wavefronts per row block
  static constexpr int kDw = D / kSplitD;                     // output dims per wavefront
  static constexpr int kDpl = kDw / 16;                       // V dims per lane (= output blocks)
  static constexpr int kQRegs = BF16 ? D / 32 : D / 16;       // 16-byte Q/K pieces per lane
  static constexpr int kLoads = kStageBytes / 16 / kThreadsC;  // 16-byte loads per thread per stage
#ifdef WMTP_COOP_PREFETCH
  static constexpr int kPrefetch = WMTP_COOP_PREFETCH;       // stages in flight
#else
  // stages in flight: about 16 KB per workgroup (two stages of 8 KB or more, four of 4 KB).
  // Measured on MI355X (verification, head_dim 128, bf16, 2 workgroups per CU): 2 stages of 8 KB
  // beat 3, 4 and 6 (more loads in flight per CU lowered the achieved bandwidth) and 1.
  static constexpr int kPrefetch = kStageBytes >= 8192 ? 2 : 4;
#endif
  static_assert(kLoads >= 1 && kStageBytes % (16 * kThreadsC) == 0, "stage must split evenly");
  static_assert(kDpl >= (BF16 ? 2 : 1), "each lane needs a pair of bf16 dims");
};

// Byte offset of 16-byte chunk `chunk` of key `key` in a staged K (tensor 0) or V (tensor 1) tile.
// K chunks are XOR-swizzled by key: the S^T operand read takes 16 keys' chunk ks*4+grp in one
// instruction, which would otherwise fall into the same banks (measured on MI355X: 28 conflict
// cycles per read unswizzled, none swizzled). bf16 V is read with transposing reads in which each
// 16-lane group takes the same 32-byte segment of four consecutive keys; its 32-byte segments are
// XOR-swizzled by (key & 7) so that eight consecutive keys' segments cover all banks. fp32 V is
// read one key row per 16 lanes and stays plain (conflict-free as it is).
template <int D, int NB, bool BF16>
__device__ __forceinline__ int coop_slot(int key, int chunk, int tensor) {
  using C = Coop<D, NB, BF16>;
  if (tensor == 0) return key * C::kRowBytes + ((chunk ^ (key & C::kSwz)) << 4);
  if constexpr (BF16) return key * C::kRowBytes + ((chunk ^ (2 * (key & C::kVSwz))) << 4);
  return key * C::kRowBytes + (chunk << 4);
}

template <int D, int NB, bool BF16, bool RING, bool FUSED>
#ifndef WMTP_COOP_WPC
#define WMTP_COOP_WPC 2
#endif
__global__ __launch_bounds__((64 * Coop<D, NB, BF16>::kWaves), WMTP_COOP_WPC)
void attn_coop_kernel(AttnArgs a, int n_splits, int n_chunks, int chunk_rows) {
  using C = Coop<D, NB, BF16>;
  typedef typename std::conditional<BF16, bf16x8_t, f32x4_t>::type QVec;
  __shared__ __attribute__((aligned(16))) char sm_tile[2][C::kStageBytes];
  request_args(a);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // row blocks of this wavefront: rb0 + 4*j, j < kRbw (NB = 8: blocks wave and wave + 4)
  const int rb0 = wave / C::kSplitD;
  const int d0 = (wave % C::kSplitD) * C::kDw;
  const int split = blockIdx.x;
  const int bhc = blockIdx.y;
  // (divisions by the call's invariant sizes as multiply-shifts: every operand is below 2^31)
  const int bh = div_of(bhc, a.div_chunks);
  const int chunk = bhc - bh * n_chunks;
  const int b = div_of(bh, a.div_kv);
  const int h = bh - b * a.n_kv_heads;
  const int G = a.div_g.d;
  const int rows = G * a.m;
  const int row_end = min(rows, chunk * chunk_rows + chunk_rows);
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const size_t head_off = (size_t)(b * a.n_kv_heads + h) * (size_t)a.capacity * C::kRowBytes;
  const char* kbase = static_cast<const char*>(a.k) + head_off;
  const char* vbase = static_cast<const char*>(a.v) + head_off;

  // query operand of this wavefront's row block. Loaded before the tile prefetch so that the
  // loads outstanding at the top of the tile loop are the same on entry and on the back edge
  // (otherwise the compiler drains every load there, once per round of kPrefetch tiles).
  // A padding row (past the last query row) loads the last real row instead of zeros: its
  // results are never written, and an unconditional load needs no wait before the prefetch.
  bool row_ok[C::kRbw];
  int row_j[C::kRbw];  // candidate index of the row
  QVec qf[C::kRbw][C::kQRegs];
#pragma unroll
  for (int j = 0; j < C::kRbw; ++j) {
    const int row = chunk * chunk_rows + (rb0 + C::kWaves * j) * 16 + r16;
    row_ok[j] = row < row_end;
    const int row_q = row_ok[j] ? row : row_end - 1;
    const int jq = div_of(row_q, a.div_g);
    const int hq = h * G + (row_q - jq * G);
    row_j[j] = jq;
    const size_t qoff = ((size_t)(b * a.m + jq) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int ks = 0; ks < C::kQRegs; ++ks)
      qf[j][ks] = __builtin_bit_cast(
          QVec, *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + qoff * C::kEB +
                                                (ks * 4 + grp) * 16));
  }
  // seq_len: read before the tile prefetch in a fused verification (the candidates' positions
  // steer its loads), else only once the prefetch is out (it only masks)
  int n = 0;
  // fused verification (contiguous cache): the m candidates at positions n .. n+m-1 are read from
  // new_k/new_v ([batch][m][n_kv_heads][head_dim]) and stored by workgroup (split 0, chunk 0)
  int fresh = 0x7fffffff;
  const char* knew = nullptr;
  const char* vnew = nullptr;
  if constexpr (FUSED) {
    n = max(a.seq_len[b], 0);
    fresh = n;
    const size_t off = ((size_t)b * a.m * a.n_kv_heads + h) * C::kRowBytes;
    knew = static_cast<const char*>(a.new_k) + off;
    vnew = static_cast<const char*>(a.new_v) + off;
  }
  // Addresses only depend on the host-side bound a.limit (>= 1), so the first tiles are requested
  // without waiting for seq_len (except in a fused verification); seq_len only masks (a tile past
  // it is computed fully masked).
  const int tiles_lim = (a.limit + kTileKeys - 1) / kTileKeys;
  const int last_lim = a.limit - 1;
  auto tile_start = [&](int i) {  // first key of the workgroup's i-th tile, clamped into range
    const int tl = split + i * n_splits;
    return (tl < tiles_lim ? tl : tiles_lim - 1) * kTileKeys;
  };

  // staging: load l of this thread is chunk q = tid + kThreadsC*l of the stage: tile q / (32*kChunks),
  // then K chunks before V chunks
  uint4 stg[C::kPrefetch][C::kLoads];
  auto load_stage = [&](uint4(&dst)[C::kLoads], int stage) {
#pragma unroll
    for (int l = 0; l < C::kLoads; ++l) {
      const int q = tid + C::kThreadsC * l;
      const int u = q / (32 * C::kChunks);  // tile of the stage
      const int tensor = (q / (16 * C::kChunks)) & 1;
      const int key = (q / C::kChunks) % 16;
      const int c = q % C::kChunks;
      const int t0 = tile_start(stage * C::kTps + u);
      const int kg = min(t0 + key, last_lim);
      const char* row = (tensor ? vbase : kbase) + (size_t)kg * C::kRowBytes;
      if constexpr (FUSED) {
        // only the last tiles can hold a candidate of this call (a workgroup-uniform test first)
        if (t0 + kTileKeys > fresh) {
          if (kg >= fresh && kg - fresh < a.m)  // a candidate: its row comes from new_k/new_v
            row = (tensor ? vnew : knew) + (size_t)(kg - fresh) * a.n_kv_heads * C::kRowBytes;
        }
      }
      dst[l] = stream_load16(row + c * 16);
    }
  };
  // Staged tiles may run past the length (the first stages are requested against the host-side
  // bound, and a workgroup's rounds end in tiles past its share). Their keys get weight 0, but
  // 0 * NaN is NaN, so a stage that reaches past `clip_last` (the last attended key, set once
  // seq_len is known) stores zeros for those keys instead (a workgroup-uniform branch, taken only
  // by such stages).
  int clip_last = 0x7fffffff;
  auto store_stage = [&](const uint4(&src)[C::kLoads], int buf, int stage) {
    const bool clip = tile_start(stage * C::kTps + C::kTps - 1) + kTileKeys - 1 > clip_last;
#pragma unroll
    for (int l = 0; l < C::kLoads; ++l) {
      const int q = tid + C::kThreadsC * l;
      const int u = q / (32 * C::kChunks);
      const int tensor = (q / (16 * C::kChunks)) & 1;
      const int key = (q / C::kChunks) % 16;
      const int c = q % C::kChunks;
      uint4 x = src[l];
      if (clip && tile_start(stage * C::kTps + u) + key > clip_last) x = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&sm_tile[buf][(2 * u + tensor) * C::kTileBytes +
                                              coop_slot<D, NB, BF16>(key, c, tensor)]) = x;
    }
  };

  // The prefetch is issued on every path (a workgroup without tiles reads clamped, valid rows) and
  // stage by stage (the scheduling barriers keep the compiler from interleaving the stages' loads):
  // the loads outstanding at the top of the tile loop are then in the same order on entry as on
  // the back edge, so the loop waits for exactly the oldest stage. (With a conditional prefetch,
  // or loads grouped by index across stages, the waits merged at the loop header let only about
  // two of the kPrefetch stages stay in flight.)
#pragma unroll
  for (int s = 0; s < C::kPrefetch; ++s) {
    load_stage(stg[s], s);
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (FUSED) {
    if (split == 0 && chunk == 0) {
      constexpr int kPieces = C::kRowBytes / 16;
      for (int i = tid; i < 2 * a.m * kPieces; i += C::kThreadsC) {
        const int tensor = i / (a.m * kPieces);
        const int j = (i / kPieces) % a.m;
        const int c = i % kPieces;
        const int64_t p = (int64_t)n + j;
        if (p >= a.capacity) continue;
        const char* src = (tensor ? vnew : knew) + (size_t)j * a.n_kv_heads * C::kRowBytes;
        char* dst = const_cast<char*>(tensor ? vbase : kbase) + (size_t)p * C::kRowBytes;
        reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
        if (a.pos && h == 0 && tensor == 0 && c == 0) a.pos[(size_t)b * a.capacity + p] = (int32_t)p;
      }
    }
    n = n <= 0x7fffffff - a.m ? n + a.m : 0x7fffffff;
  } else {
    n = max(a.seq_len[b], 0);
  }
  const RingMask rm = ring_mask(a, n);
  n = min(n, a.limit);
  const int last = n - 1;
  clip_last = last;
  const int tiles = (n + kTileKeys - 1) / kTileKeys;
  const int my_tiles = split < tiles ? (tiles - split + n_splits - 1) / n_splits : 0;
  const int my_stages = (my_tiles + C::kTps - 1) / C::kTps;
  int last_visible[C::kRbw];
#pragma unroll
  for (int j = 0; j < C::kRbw; ++j)
    last_visible[j] = (a.mode == kModeVerify) ? (n - a.m + row_j[j]) : (n - 1);
  // the last key every row of the workgroup may attend (candidate 0 sees the fewest)
  const int vis_all = min(last, (a.mode == kModeVerify) ? (n - a.m) : (n - 1));

  const float scale_log2 = a.sm_scale * kLog2e;
  float m_ref[C::kRbw];   // reference max (log2 units), shared by the row's four lanes
  float l_lane[C::kRbw];  // this lane's share of the running sum
  f32x4_t o[C::kRbw][C::kDpl];
#pragma unroll
  for (int j = 0; j < C::kRbw; ++j) {
    m_ref[j] = -INFINITY;
    l_lane[j] = 0.f;
#pragma unroll
    for (int e = 0; e < C::kDpl; ++e) o[j][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // one 16-key tile: K at kt, V at kt + kTileBytes (swizzled LDS layout); i = the workgroup's
  // tile index (tiles past its share are computed fully masked)
  auto tile_step = [&](const char* kt, int i) {
    const bool live = i < my_tiles;  // workgroup-uniform
    const int t0 = tile_start(i);
    const char* vt = kt + C::kTileBytes;
    // ---- S^T (16 keys x 16 rows) for each of this wavefront's row blocks
    f32x4_t sacc[C::kRbw];
#pragma unroll
    for (int j = 0; j < C::kRbw; ++j) sacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::kQRegs; ++ks) {
      const uint4 kv =
          *reinterpret_cast<const uint4*>(kt + coop_slot<D, NB, BF16>(r16, ks * 4 + grp, 0));
#pragma unroll
      for (int j = 0; j < C::kRbw; ++j) {
        if constexpr (BF16) {
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                            qf[j][ks], sacc[j], 0, 0, 0);
        } else {
          const float4 kf = __builtin_bit_cast(float4, kv);
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x, qf[j][ks][0], sacc[j], 0, 0, 0);
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.y, qf[j][ks][1], sacc[j], 0, 0, 0);
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.z, qf[j][ks][2], sacc[j], 0, 0, 0);
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.w, qf[j][ks][3], sacc[j], 0, 0, 0);
        }
      }
    }

    // ---- softmax with a lazily moved reference max (as in the split kernel)
    float p[C::kRbw][4];
#pragma unroll
    for (int j = 0; j < C::kRbw; ++j) {
      const int vis = live ? min(last, last_visible[j]) : -1;
      float sc[4];
      float mx = -INFINITY;
      if (!RING && live && t0 + kTileKeys - 1 <= vis_all) {  // workgroup-uniform: none masked
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sc[t] = sacc[j][t] * scale_log2;
          mx = fmaxf(mx, sc[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int key = t0 + 4 * grp + t;
          const bool ok = key <= vis && (!RING || rm.attended(key));
          sc[t] = ok ? sacc[j][t] * scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[t]);
        }
      }
      if (__ballot(mx > m_ref[j] + kRescaleLog2)) {  // lane-local test first, as in the split kernel
        mx = xgroup_max(mx);
        const bool moved = mx > m_ref[j] + kRescaleLog2;
        const float alpha = moved ? __builtin_amdgcn_exp2f(m_ref[j] - mx) : 1.f;
        l_lane[j] *= alpha;
#pragma unroll
        for (int e = 0; e < C::kDpl; ++e) o[j][e] *= alpha;
        m_ref[j] = moved ? mx : m_ref[j];
      }
      const float m_use = (m_ref[j] == -INFINITY) ? 0.f : m_ref[j];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        p[j][t] = __builtin_amdgcn_exp2f(sc[t] - m_use);
        l_lane[j] += p[j][t];
      }
    }

    // ---- O^T (this wavefront's dims) += V^T . P^T, one V operand shared by the row blocks
    if constexpr (BF16) {
      // Block e covers dims d0 + 16e .. +15. The V^T operand (lane (r16, grp): keys 4*grp .. +3
      // of dim d0 + 16e + r16) comes from one transposing LDS read per block: within each 16-lane
      // group, lane 4j + q addresses the 8 bytes of key 4*grp + j at dims d0 + 16e + 4q .. +3,
      // and lane i receives element i % 4 of what lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4 address.
      s16x4_t pop[C::kRbw];
#pragma unroll
      for (int j = 0; j < C::kRbw; ++j) {
        const bf16x4_t pb =
            __builtin_convertvector(f32x4_t{p[j][0], p[j][1], p[j][2], p[j][3]}, bf16x4_t);
        pop[j] = __builtin_bit_cast(s16x4_t, pb);
      }
      const int vkey = 4 * grp + (r16 >> 2);
#pragma unroll
      for (int e = 0; e < C::kDpl; ++e) {
        const int c = ((d0 + 16 * e) >> 3) + ((r16 >> 1) & 1);
        const char* src = vt + coop_slot<D, NB, BF16>(vkey, c, 1) + (r16 & 1) * 8;
        typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
        const s16x4_t vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(__attribute__((address_space(3))) const char*)src);
#pragma unroll
        for (int j = 0; j < C::kRbw; ++j)
          o[j][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop[j], o[j][e], 0, 0, 0);
      }
    } else {
      // lane r16 owns dims d0 + kDpl*r16 + e: one key row's kDpl consecutive dims per lane
      uint32_t vw[4][C::kDpl];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const char* src = vt + (4 * grp + t) * C::kRowBytes + (d0 + C::kDpl * r16) * C::kEB;
#pragma unroll
        for (int w = 0; w < C::kDpl; w += (C::kDpl >= 4 ? 4 : C::kDpl)) {
          if constexpr (C::kDpl >= 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(src + 4 * w);
            vw[t][w] = x.x; vw[t][w + 1] = x.y; vw[t][w + 2] = x.z; vw[t][w + 3] = x.w;
          } else if constexpr (C::kDpl == 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(src);
            vw[t][0] = x.x; vw[t][1] = x.y;
          } else {
            vw[t][0] = *reinterpret_cast<const uint32_t*>(src);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < C::kRbw; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < C::kDpl; ++e)
            o[j][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, vw[u][e]),
                                                           p[j][u], o[j][e], 0, 0, 0);
    }
  };

  // A wavefront whose one row block lies wholly past the chunk's last row (padding up to the
  // planned block count, e.g. 80 rows run as 8 blocks) stages its share of the tiles and meets the
  // barriers but computes nothing.
  const bool wave_live =
      C::kRbw > 1 || __builtin_amdgcn_readfirstlane(rb0 * 16) < row_end - chunk * chunk_rows;
  // Rounds of exactly kPrefetch tiles with no early exit: tiles past the workgroup's share are
  // computed fully masked. The straight-line round lets the compiler wait for exactly the oldest
  // staged tile (an early exit inside the round makes it drain every load at the round start).
  for (int base = 0; base < my_stages; base += C::kPrefetch) {
#pragma unroll
    for (int s = 0; s < C::kPrefetch; ++s) {
      const int st = base + s;
      const int buf = st & 1;
      store_stage(stg[s], buf, st);
      load_stage(stg[s], st + C::kPrefetch);
      __syncthreads();  // stage st visible; every wavefront is done with stage st-1's buffer
#pragma unroll
      for (int u = 0; u < C::kTps; ++u)
        if (wave_live) tile_step(sm_tile[buf] + 2 * u * C::kTileBytes, st * C::kTps + u);
    }
  }

  // ---- this wavefront's part of the workgroup's partial
  const size_t part = (size_t)bhc * a.part_stride + a.part_offset + split;
  constexpr int kRows = 16 * NB;
#pragma unroll
  for (int j = 0; j < C::kRbw; ++j) {
    const float l_row = xgroup_sum(l_lane[j]);
    if (!row_ok[j]) continue;
    const int rloc = (rb0 + C::kWaves * j) * 16 + r16;
    float* dst = a.ws_o + (part * kRows + rloc) * D + d0;
    if constexpr (BF16) {
      // lane (r16, grp) holds O^T rows 4*grp + t of block e: dims d0 + 16e + 4*grp + t
#pragma unroll
      for (int e = 0; e < C::kDpl; ++e)
        *reinterpret_cast<float4*>(dst + 16 * e + 4 * grp) =
            make_float4(o[j][e][0], o[j][e][1], o[j][e][2], o[j][e][3]);
    } else {
      // lane (r16, grp) holds O^T rows 4*grp + t of block e: dim d0 + kDpl*(4*grp + t) + e
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float* d = dst + C::kDpl * (4 * grp + t);
        if constexpr (C::kDpl >= 4) {
#pragma unroll
          for (int e = 0; e < C::kDpl; e += 4)
            *reinterpret_cast<float4*>(d + e) =
                make_float4(o[j][e][t], o[j][e + 1][t], o[j][e + 2][t], o[j][e + 3][t]);
        } else {
#pragma unroll
          for (int e = 0; e < C::kDpl; ++e) d[e] = o[j][e][t];
        }
      }
    }
    if (d0 == 0 && grp == 0)
      *reinterpret_cast<float2*>(a.ws_ml + (part * kRows + rloc) * 2) = make_float2(m_ref[j], l_row);
  }
}

// One workgroup per (output row, 4*COLS dims). COLS threads cover the dims as float4 columns;
// 256/COLS lanes of splits stride over the partials in one online pass (each lane keeps its own
// running max and rescales), a batch of BATCH independent loads per lane (sized to the split
// count, up to 256 splits in one batch); the lanes then combine with the same rescaling rule, by
// shuffles inside each wavefront and through LDS across the four. Measured on MI355X: 8 columns (twice the workgroups, half the loads per
// lane) are as fast or faster up to 256 splits per row (the draft steps' 65-128, verification's
// 256); 16 columns take larger split counts in one batch.
template <int D, int COLS, int BATCH>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int n_splits, int n_chunks,
                                                    int chunk_rows, int nr) {
  constexpr int kCols = COLS;
  constexpr int kSplitLanes = 256 / kCols;
  constexpr int kBatch = BATCH;
  __shared__ float red_m[256];
  __shared__ float4 red_o[256];
  __shared__ float red_l[256];
  request_args(a);

  // index arithmetic in unsigned ints (all values are nonnegative), divisions by the call's
  // invariant sizes as multiply-shifts
  const unsigned row_id = blockIdx.x;  // ((b * m + j) * Hq + hq)
  const int dim0 = blockIdx.y * (4 * kCols);
  const unsigned nq = a.n_q_heads, nkv = a.n_kv_heads, um = a.m, crows = chunk_rows;
  const unsigned bj = div_of(row_id, a.div_hq);
  const unsigned hq = row_id - bj * nq;
  const unsigned b = div_of(bj, a.div_m);
  const unsigned j = bj - b * um;
  const unsigned G = a.div_g.d;
  const unsigned h = div_of(hq, a.div_g);
  const unsigned row = j * G + (hq - h * G);
  const unsigned chunk = div_of(row, a.div_crows);
  const int rloc = row - chunk * crows;
  const size_t base = ((size_t)(b * nkv + h) * n_chunks + chunk) * n_splits;
  const int rows16 = 16 * nr;
  const int tid = threadIdx.x;
  const int col = tid % kCols;
  const int sl = tid / kCols;
  auto ml_at = [&](int s) {
    return *reinterpret_cast<const float2*>(a.ws_ml + ((base + s) * rows16 + rloc) * 2);
  };
  auto o_at = [&](int s) {
    return *reinterpret_cast<const float4*>(a.ws_o + ((base + s) * rows16 + rloc) * D + dim0 +
                                            col * 4);
  };

  // running state of this lane: sum_s 2^(m_s - M) (o_s, l_s) over the partials seen so far
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto absorb = [&](float2 ml, float4 x) {
    // an empty partial (no attended key: max -inf, sum 0) is skipped; a NaN partial is not, so a
    // NaN among the attended keys reaches the output as it does in exact arithmetic
    if (ml.y == 0.f) return;
    if (ml.x > M) {
      const float c = __builtin_amdgcn_exp2f(M - ml.x);  // 0 while M is -inf
      L *= c; acc.x *= c; acc.y *= c; acc.z *= c; acc.w *= c;
      M = ml.x;
    }
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    L += w * ml.y;
    acc.x += w * x.x; acc.y += w * x.y; acc.z += w * x.z; acc.w += w * x.w;
  };
  // batches of kBatch partials per lane, all loads of a batch in flight together (one batch covers
  // up to 256 splits); indices past the last split re-read it and are not absorbed
  for (int s0 = sl; s0 < n_splits; s0 += kBatch * kSplitLanes) {
    float2 ml[kBatch];
    float4 x[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int si = min(s0 + i * kSplitLanes, n_splits - 1);
      ml[i] = ml_at(si);
      x[i] = o_at(si);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s0 + i * kSplitLanes < n_splits) absorb(ml[i], x[i]);
  }

  // combine (M, L, acc) over the split lanes: first inside the wavefront (lanes that differ in
  // the split bits of the lane index, by cross-lane shuffles), then the four wavefronts' results
  // through LDS with one barrier
  auto combine = [&](float m2, float l2, float4 x2) {
    const float mm = fmaxf(M, m2);
    const float mu = (mm == -INFINITY) ? 0.f : mm;
    const float c1 = __builtin_amdgcn_exp2f(M - mu), c2 = __builtin_amdgcn_exp2f(m2 - mu);
    M = mm;
    L = c1 * L + c2 * l2;
    acc = make_float4(c1 * acc.x + c2 * x2.x, c1 * acc.y + c2 * x2.y, c1 * acc.z + c2 * x2.z,
                      c1 * acc.w + c2 * x2.w);
  };
#pragma unroll
  for (int off = kCols; off < 64; off <<= 1)
    combine(__shfl_xor(M, off), __shfl_xor(L, off),
            make_float4(__shfl_xor(acc.x, off), __shfl_xor(acc.y, off), __shfl_xor(acc.z, off),
                        __shfl_xor(acc.w, off)));
  const int wave = tid >> 6;
  if ((tid & 63) < kCols) {
    red_m[wave * kCols + col] = M;
    red_l[wave * kCols + col] = L;
    red_o[wave * kCols + col] = acc;
  }
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w)
      combine(red_m[w * kCols + col], red_l[w * kCols + col], red_o[w * kCols + col]);
    red_m[col] = M;
    red_l[col] = L;
    red_o[col] = acc;
  }
  if (a.new_k && j == 0 && hq == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    // fused step: every attention workgroup has finished, so the length can advance now (by the
    // m tokens the call appended)
    int32_t* len_p = const_cast<int32_t*>(a.seq_len);  // the caller's (mutable) lengths
    const int32_t len = *(len_p + b);
    const int32_t base = len < 0 ? 0 : len;
    len_p[b] = base <= 0x7fffffff - a.m ? base + a.m : 0x7fffffff;
  }
  if (sl == 0) {
    const float Lt = red_l[col];
    const float4 r = red_o[col];
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    if (Lt != 0.f) {  // else nothing was attended: out = 0, lse = -inf (NaN propagates)
      const float inv = 1.f / Lt;
      res = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    }
    *reinterpret_cast<float4*>(a.out + (size_t)row_id * D + dim0 + col * 4) = res;
    if (col == 0 && blockIdx.y == 0 && a.lse)
      a.lse[row_id] = (Lt != 0.f) ? (red_m[0] + log2f(Lt)) * kLn2 : -INFINITY;
  }
}

template <int D, bool BF16>
hipError_t launch_split(const AttnArgs& a, const SplitPlan& p, hipStream_t stream) {
  dim3 grid(p.n_splits, a.batch * a.n_kv_heads * p.n_chunks);
  dim3 block(kThreads);
  // row blocks beyond the register budget of (D, dtype) are never planned (rows_cap)
  constexpr int kMaxNr = BF16 ? (D == 256 ? 2 : 4) : (D == 64 ? 4 : (D == 128 ? 2 : 1));
  if (p.nr < 1 || p.nr > kMaxNr) return hipErrorInvalidValue;
  const bool ring = ring_masked(a);
  const bool fused = a.new_k != nullptr;
  if (p.q_lds && p.nr != 1) return hipErrorInvalidValue;  // planned for one row block only
#define WMTP_SPLIT1(RINGV, FUSEDV)                                                                      \
  do {                                                                                                 \
    if (p.q_lds)                                                                                       \
      attn_split_kernel<D, 1, BF16, RINGV, FUSEDV, true><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); \
    else                                                                                               \
      attn_split_kernel<D, 1, BF16, RINGV, FUSEDV, false><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); \
  } while (0)
  if (ring || fused) {
    // draft steps have one query token: G <= 16 rows, one row block
    if (p.nr != 1) return hipErrorInvalidValue;
    if (ring && fused) WMTP_SPLIT1(true, true);
    else if (ring) WMTP_SPLIT1(true, false);
    else WMTP_SPLIT1(false, true);
  } else {
    switch (p.nr) {
      case 1: WMTP_SPLIT1(false, false); break;
      case 2: if constexpr (kMaxNr >= 2) attn_split_kernel<D, 2, BF16, false, false, false><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); break;
      case 3: if constexpr (kMaxNr >= 3) attn_split_kernel<D, 3, BF16, false, false, false><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); break;
      default: if constexpr (kMaxNr >= 4) attn_split_kernel<D, 4, BF16, false, false, false><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); break;
    }
  }
#undef WMTP_SPLIT1
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_coop(const AttnArgs& a, const SplitPlan& p, hipStream_t stream) {
  dim3 grid(p.n_splits, a.batch * a.n_kv_heads * p.n_chunks);
  const bool ring = ring_masked(a);
  const bool fused = a.new_k != nullptr;  // fused verification: contiguous cache, one row chunk
  if (ring && fused) return hipErrorInvalidValue;
#define WMTP_COOP_LAUNCH(NBV)                                                                          \
  do {                                                                                                 \
    const dim3 block(64 * Coop<D, NBV, BF16>::kWaves);                                                 \
    if (ring) attn_coop_kernel<D, NBV, BF16, true, false><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); \
    else if (fused) attn_coop_kernel<D, NBV, BF16, false, true><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); \
    else attn_coop_kernel<D, NBV, BF16, false, false><<<grid, block, 0, stream>>>(a, p.n_splits, p.n_chunks, p.chunk_rows); \
  } while (0)
  switch (p.nr) {
    case 1:
      if constexpr (!(BF16 && D == 64)) WMTP_COOP_LAUNCH(1);
      break;
    case 2:
      WMTP_COOP_LAUNCH(2);
      break;
    case 4:
      if constexpr (BF16 || D != 256) WMTP_COOP_LAUNCH(4);
      break;
    case 8:
      if constexpr (BF16 && D <= 128) WMTP_COOP_LAUNCH(8);
      else return hipErrorInvalidValue;
      break;
    default: return hipErrorInvalidValue;
  }
#undef WMTP_COOP_LAUNCH
  return hipGetLastError();
}

}  // namespace

#ifndef WMTP_MIN_TILES_PER_WAVE
#define WMTP_MIN_TILES_PER_WAVE 1
#endif
constexpr long long kMinTilesPerWave = WMTP_MIN_TILES_PER_WAVE;
constexpr int kSplitMaxRows = 48;  // most query rows per KV head on the key-split kernel

// Largest row chunk whose Q operand and O accumulators fit the register file beside the K/V tiles.
static int rows_cap(int dtype, int head_dim) {
  if (dtype == WMTP_BF16) return head_dim == 256 ? 32 : 64;
  return head_dim == 64 ? 64 : (head_dim == 128 ? 32 : 16);
}

bool make_plan_for(int batch, int n_q_heads, int n_kv_heads, int head_dim, int m,
                   int max_seq_len, int dtype, SplitPlan* p) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads) return false;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return false;
  if (m < 1 || m > kMaxM || max_seq_len < 1 || max_seq_len > kMaxCapacity) return false;
  p->G = n_q_heads / n_kv_heads;
  p->rows = p->G * m;
  // Key-split kernel for one row block, and for a verification whose rows fit one of its row
  // chunks in at most three 16-row blocks; cooperative tiles beyond. Each kernel runs with the
  // workgroup count measured best for it. Measured on MI355X (verification at 256K-1M keys, steady
  // state): the key-split kernel wins at 24-48 rows by 8-24% (bf16 head_dim 64/128/256, fp32
  // 64/128; e.g. bf16 d128 at 32 rows 154 vs 167 us) and loses at 64 rows (four blocks leave no
  // register room for its prefetch: 208 vs 173 us) and wherever the rows need a second chunk (the
  // cache is then read twice). Draft steps (one query token) keep the cooperative kernel above 16
  // rows: the key-split kernel's ring-masked and fused forms take one row block.
  const bool split_rows =
      p->rows <= 16 || (m > 1 && p->rows <= std::min(rows_cap(dtype, head_dim), kSplitMaxRows));
  p->coop = kAllowCoop && !split_rows;
  const int target_blocks = p->coop ? kTargetBlocksCoop : kTargetBlocksSplit;
  // row blocks per cooperative workgroup within the register budget: eight (one per wavefront on
  // eight wavefronts, or two per wavefront on four) for bf16 up to head_dim 128, two for fp32 at
  // head_dim 256, four otherwise
  const int coop_cap = (dtype == WMTP_BF16 && head_dim <= 128) ? 2 * kWavesPerBlock * 16
                       : (dtype == WMTP_F32 && head_dim == 256) ? 32 : kWavesPerBlock * 16;
  const int cap = p->coop ? coop_cap : rows_cap(dtype, head_dim);
  p->chunk_rows = p->rows < cap ? p->rows : cap;
  p->n_chunks = (p->rows + p->chunk_rows - 1) / p->chunk_rows;
  p->nr = (p->chunk_rows + 15) / 16;
  if (p->coop) {
    // row blocks per workgroup: 1, 2, 4 (the wavefronts split the rest by dims) or 8 (two per
    // wavefront); a bf16 lane needs at least two dims, so head_dim 64 keeps two row blocks
    if (p->nr == 3) p->nr = 4;
    if (p->nr > 4) p->nr = 8;
    if (dtype == WMTP_BF16 && head_dim == 64 && p->nr < 2) p->nr = 2;
  }
  const long long bhc = (long long)batch * n_kv_heads * p->n_chunks;
  if (bhc > 65535) return false;  // one grid row per (sequence, KV head, row chunk)
  const long long tiles_per_seq = ((long long)max_seq_len + kTileKeys - 1) / kTileKeys;
  // about target_blocks workgroups in all, but at least kMinTilesPerWave tiles per wavefront
  long long blocks = (bhc * tiles_per_seq + kWavesPerBlock * kMinTilesPerWave - 1) /
                     (kWavesPerBlock * kMinTilesPerWave);
  if (blocks > target_blocks) blocks = target_blocks;
  long long per = (blocks + bhc - 1) / bhc;
  const long long cap_per =
      (tiles_per_seq + kWavesPerBlock * kMinTilesPerWave - 1) / (kWavesPerBlock * kMinTilesPerWave);
  if (per > cap_per) per = cap_per;
  if (per < 1) per = 1;
  p->n_splits = (int)per;
  // A short read (the windowed draft step: a few thousand keys per KV head) fills fewer workgroups
  // than the target, each of about one tile per wavefront; it is latency-bound. Its query operand
  // is loaded once per workgroup into LDS instead of once per wavefront: measured on MI355X at the
  // million-token draft shapes, a quarter fewer bytes through each CU's address unit bring the
  // tiles in 0.8 us earlier (windowed call 9.65 -> 9.2 us, graph-replayed).
  p->q_lds = !p->coop && p->nr == 1 && bhc * cap_per < target_blocks;
  p->ws_o_floats = (size_t)bhc * p->n_splits * 16 * p->nr * head_dim;
  p->ws_ml_floats = (size_t)bhc * p->n_splits * 16 * p->nr * 2;
  return true;
}

// The kernels' divisors for the sizes of `a` and the plan.
static AttnArgs with_divisors(const AttnArgs& a, const SplitPlan& p) {
  AttnArgs b = a;
  b.div_hq = make_fastdiv(a.n_q_heads);
  b.div_kv = make_fastdiv(a.n_kv_heads);
  b.div_g = make_fastdiv(a.n_q_heads / a.n_kv_heads);
  b.div_m = make_fastdiv(a.m);
  b.div_chunks = make_fastdiv(p.n_chunks);
  b.div_crows = make_fastdiv(p.chunk_rows);
  return b;
}

template <int D>
hipError_t launch_merge(const AttnArgs& a, const SplitPlan& p, int total_splits, hipStream_t stream) {
  const unsigned rows = a.batch * a.m * a.n_q_heads;
  // loads per split lane sized to the split count (a lane's slots past the last split would only
  // re-read it): 8 columns x 32 split lanes x 1-8 loads up to 256 splits, 16 x 16 x 16 beyond
  const dim3 g8(rows, D / 32), g16(rows, D / 64), blk(256);
  if (total_splits > 256)
    merge_kernel<D, 16, 16><<<g16, blk, 0, stream>>>(a, total_splits, p.n_chunks, p.chunk_rows, p.nr);
  else if (total_splits > 128)
    merge_kernel<D, 8, 8><<<g8, blk, 0, stream>>>(a, total_splits, p.n_chunks, p.chunk_rows, p.nr);
  else if (total_splits > 64)
    merge_kernel<D, 8, 4><<<g8, blk, 0, stream>>>(a, total_splits, p.n_chunks, p.chunk_rows, p.nr);
  else if (total_splits > 32)
    merge_kernel<D, 8, 2><<<g8, blk, 0, stream>>>(a, total_splits, p.n_chunks, p.chunk_rows, p.nr);
  else
    merge_kernel<D, 8, 1><<<g8, blk, 0, stream>>>(a, total_splits, p.n_chunks, p.chunk_rows, p.nr);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& args, const SplitPlan& p, int total_splits, hipStream_t stream) {
  const AttnArgs a = with_divisors(args, p);
  switch (a.head_dim) {
    case 64: return launch_merge<64>(a, p, total_splits, stream);
    case 128: return launch_merge<128>(a, p, total_splits, stream);
    case 256: return launch_merge<256>(a, p, total_splits, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnArgs& a, const SplitPlan& p, int dtype, hipStream_t stream) {
  hipError_t e = launch_partials(a, p, dtype, stream);
  if (e != hipSuccess) return e;
  return launch_merge(a, p, a.part_stride, stream);
}

hipError_t launch_partials(const AttnArgs& args, const SplitPlan& p, int dtype, hipStream_t stream) {
  const AttnArgs a = with_divisors(args, p);
  const bool bf16 = dtype == WMTP_BF16;
  if (p.coop) {
    switch (a.head_dim) {
      case 64: return bf16 ? launch_coop<64, true>(a, p, stream) : launch_coop<64, false>(a, p, stream);
      case 128: return bf16 ? launch_coop<128, true>(a, p, stream) : launch_coop<128, false>(a, p, stream);
      case 256: return bf16 ? launch_coop<256, true>(a, p, stream) : launch_coop<256, false>(a, p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.head_dim) {
    case 64: return bf16 ? launch_split<64, true>(a, p, stream) : launch_split<64, false>(a, p, stream);
    case 128: return bf16 ? launch_split<128, true>(a, p, stream) : launch_split<128, false>(a, p, stream);
    case 256: return bf16 ? launch_split<256, true>(a, p, stream) : launch_split<256, false>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp
