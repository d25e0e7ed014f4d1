// GQA decode step on the gfx950 matrix cores (bfloat16 or IEEE half in, float32
// accumulate; below, "16-bit" is whichever of the two the call uses).
//
// Definition: fogdragon CSDN blog, section "KV Cache" (append, then
// softmax(scale * q.K) over the cached positions and a weighted sum of V);
// GQA paper section 2.2 (n_rep = H/G query heads share one K/V head).
//
// Work unit: one workgroup of 1, 2 or 4 waves per (sequence b, K/V head g,
// split s).  The group's n_rep query heads are the 16 columns of the
// matrix-core tiles (padded with zero queries), so every cached K/V row is read
// from HBM once and used by all heads of its group (a group of 32 or more
// queries may instead be run as work groups of 16 that read the same K/V
// head, the repeat coming mostly from the last-level cache):
//
//   scores  S^T[key][head] = K[key][:] . Q[head][:]     16x16x32 16-bit MFMA,
//           A = 16 keys x 32 dims read from the wave's LDS copy of the K
//           tile (loaded as whole contiguous rows, 1 KB per instruction),
//           B = the group's queries (registers, loaded once)
//   softmax online, base 2 (hardware exp2), float32; the weights are rounded
//           to the 16-bit format and the normaliser sums the rounded weights
//           (so constant V is exact)
//   output  O^T[dim][head] += V^T[dim][key] P^T[key][head]   16x16x32 MFMA,
//           A = V^T read with transposing LDS loads from a per-wave copy of
//           the 32-row V tile, B = the weights, already in the right lanes
//           after the scores
//
// Each wave walks its own 32-position tiles of the split (tile t goes to wave
// t mod waves) with one tile in flight: the next tile's loads go out as soon
// as this tile's K and V rows are in LDS (at d = 128, K's as soon as K is),
// and land during its scores, softmax and weighted sum.  (Two tiles in
// flight per wave measured 5-17% slower, as did 2, 3, 5, 6 or 8 waves: four
// waves with one 16 KB tile each, 64 KB per compute unit, is the point past
// which more requests only lengthen each one's round trip.  K loaded straight
// into the MFMA's register layout -- 64 bytes of each of 16 rows per load
// instruction instead of 1 KB of contiguous rows -- measured 2-6% slower.)
// The waves merge (max, sum, output) through LDS.  With several
// splits, each workgroup writes its partial (max, sum, output) per head; the
// last workgroup of a (b, g) to finish -- found with a counter in the
// workspace header, which it resets -- merges the partials (log-sum-exp) and
// writes the output, so one launch does the whole step.  Positions at or
// beyond the sequence length are never loaded (the buffer loads end there and
// return zeros): their K rows are zero, their scores are set to -inf before
// the softmax and their V rows are zero, so cache contents there (NaN
// included) cannot reach the arithmetic.

#include "device_common.h"
#include "internal.h"

#include <type_traits>

namespace gqa {
namespace {

constexpr int kKT = 32;        // positions per wave step
constexpr int kMaxWaves = 4;

template <int D>
struct Cfg {
  static constexpr int kSteps = D / 32;           // MFMA k-steps over the head dimension
  static constexpr int kColBlocks = D / 16;       // 16-wide output column blocks
  static constexpr int kChunks = D / 8;           // 16-byte chunks per cached row
  static constexpr int kTileLoads = kKT * kChunks / 64;   // 64-lane 16-byte loads per K or V tile
  static constexpr int kPitch = D * 2 + 32;       // LDS bytes per V row (transposing reads hit distinct banks)
  static constexpr int kKBytes = kKT * D * 2;     // LDS bytes per K tile (rows unpadded, chunks permuted)
  static constexpr int kWaveLds = kKT * kPitch + kKBytes;
  static constexpr int kMergeRow = D + 4;         // floats per head row in the merge area
  static constexpr int kMergeBytes = (kMaxWaves * 16 * kMergeRow + 2 * kMaxWaves * 16) * 4;
  static constexpr int kLds = kMaxWaves * kWaveLds > kMergeBytes ? kMaxWaves * kWaveLds : kMergeBytes;
};

// K tile rows in LDS: 16-byte chunk c of row r at position c ^ kswz(r)
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lanes 4e..4e+3 each address 4 consecutive 16-bit values of row e of
// a 4 x 16 block, and lane i receives column i of the 4 rows.
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(const_cast<char*>(p)));
}

// 16x16x32 MFMA on raw 16-bit operands: bfloat16 or IEEE half (DT).
template <int DT>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other).  They are written and read with buffer instructions carrying the
// device-coherence bit (sc1) -- the same access an agent-scope relaxed atomic
// makes, but 16 bytes wide and free to overlap -- so no device-wide cache
// writeback or invalidate is needed.  A buffer load past the end of its
// resource returns zeros.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kDeviceCoherent = 16;    // cache-policy bit sc1
constexpr int kNonTemporal = 2;        // cache-policy bit nt (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Split partials of one (b, g) unit: part_o[b][h][s][D] and part_ml[b][h][s][2]
// for the group's n_rep heads h are contiguous, so one buffer resource --
// the same for the whole workgroup, as buffer instructions require (a
// per-lane resource would make the compiler serialise every access over the
// distinct values) -- covers all of them.
template <int D>
struct UnitPartials {
  __amdgpu_buffer_rsrc_t o, ml;
  __device__ UnitPartials(const DecodeProblem& p, int b, int g) {
    const int64_t first = (int64_t(b) * p.H + int64_t(g) * p.n_rep) * p.num_splits;
    const uint32_t n = uint32_t(p.n_rep) * uint32_t(p.num_splits);
    o = rsrc(p.part_o + first * D, n * uint32_t(D * 4));
    ml = rsrc(p.part_ml + first * 2, n * 8u);
  }
};

// Log-sum-exp merge of the ns split partials of head hl (within the group)
// and 8-column chunk c8 of sequence b, written to out.  Splits are read NB at
// a time (NB = 2, 4 or 8, the smallest batch that holds ns, so no load goes to
// a slot this call has no split for) with all their loads in flight together;
// the running maximum is rescaled per batch.
template <int D, int DT, int NB>
__device__ __forceinline__ void merge_item(const DecodeProblem& p, const UnitPartials<D>& up, int b, int ns,
                                           int g, int hl, int c8) {
  using H16 = Half16<DT>;
  const int S = p.num_splits;
  float M = -INFINITY, L = 0.f;
  f32x4_t Oa = {0.f, 0.f, 0.f, 0.f}, Ob = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int s0 = 0; s0 < ns; s0 += NB) {
    u32x2_t ml[NB];
    u32x4_t oa[NB], ob[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int pr = hl * S + s0 + u;
      ml[u] = __builtin_amdgcn_raw_buffer_load_b64(up.ml, pr * 8, 0, kDeviceCoherent);
      oa[u] = __builtin_amdgcn_raw_buffer_load_b128(up.o, pr * (D * 4) + c8 * 32, 0, kDeviceCoherent);
      ob[u] = __builtin_amdgcn_raw_buffer_load_b128(up.o, pr * (D * 4) + c8 * 32 + 16, 0, kDeviceCoherent);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (s0 + u >= ns) ml[u][1] = 0u;             // not a split of this call: skipped
    float cm = M;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (__uint_as_float(ml[u][1]) > 0.f) cm = fmaxf(cm, __uint_as_float(ml[u][0]));
    if (cm == -INFINITY) continue;               // nothing seen yet
    const float f0 = __builtin_amdgcn_exp2f(M - cm);   // 0 while M is -inf
    L *= f0;
    Oa *= f0;
    Ob *= f0;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float lu = __uint_as_float(ml[u][1]);
      // Slots of splits that did not run in this call (or saw nothing) hold
      // stale bytes -- possibly inf or NaN -- so they are selected away, never
      // multiplied by zero.
      if (lu > 0.f) {
        const float f = __builtin_amdgcn_exp2f(__uint_as_float(ml[u][0]) - cm);
        L = fmaf(lu, f, L);
        Oa += f * __builtin_bit_cast(f32x4_t, oa[u]);
        Ob += f * __builtin_bit_cast(f32x4_t, ob[u]);
      }
    }
    M = cm;
  }
  const float inv = L > 0.f ? __builtin_amdgcn_rcpf(L) : 0.f;
  st16(p.out + (int64_t(b) * p.hm.o_heads + p.hm.o_head(g, hl)) * D + c8 * 8,
       u32x4_t{H16::pack2(Oa[0] * inv, Oa[1] * inv), H16::pack2(Oa[2] * inv, Oa[3] * inv),
               H16::pack2(Ob[0] * inv, Ob[1] * inv), H16::pack2(Ob[2] * inv, Ob[3] * inv)});
}

// Phase timestamps of the measurement build (libgqa_timeline.so): thread 0
// of each workgroup writes the 100 MHz device clock at the start, when the
// sequence length is known, after its first tile, at the end of its tile loop,
// once its partial is stored (or its output written), once its arrival is
// counted, and at its end; slot 7 is the XCD it ran on.  Nothing is recorded
// in the library build.
#ifdef GQA_DECODE_TIMELINE
#define GQA_PHASE(k)                                                                           \
  do {                                                                                         \
    if (threadIdx.x == 0 && p.timeline != nullptr)                                             \
      p.timeline[(blockIdx.x + int64_t(blockIdx.y) * gridDim.x) * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define GQA_PHASE(k) \
  do {               \
  } while (0)
#endif

template <int D, int NHB, int DT, bool APPEND>
__global__ __launch_bounds__(256, NHB == 1 ? 2 : 1) void decode_mfma_kernel(DecodeProblem p) {
  using C = Cfg<D>;
  using H16 = Half16<DT>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLds];
  __shared__ int s_last;

  GQA_PHASE(0);
#ifdef GQA_DECODE_TIMELINE
  if (threadIdx.x == 0 && p.timeline != nullptr)
    p.timeline[(blockIdx.x + int64_t(blockIdx.y) * gridDim.x) * 8 + 7] =
        __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11));
#endif
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nw = blockDim.x >> 6;
  const int lo = lane & 15;
  const int hi = lane >> 4;

  // Split-major order: consecutive workgroups take the same split of
  // consecutive (b, g) units.  Workgroups are spread over the XCDs round-robin
  // by index, so every XCD gets an even share of each split index (with
  // ragged lengths the late splits are the ones that are often empty), and
  // the first splits, which are never empty, start first.
  // Work group g (its n_rep queries; kv_div work groups share a K/V head when
  // a group has more than 16 queries) of sequence b reads K/V head g_kv.  The
  // grid is (splits x sequences x K/V heads, kv_div): the hardware deals
  // workgroups to the 8 XCDs round-robin by linear index, so the kv_div work
  // groups of one K/V head, a whole grid row apart, run on one XCD whenever
  // the row length is a multiple of 8, and the second read of every K/V row
  // is served by that XCD's L2 instead of HBM.
  const int S = p.num_splits;
  const int G_kv = p.G / p.kv_div;
  const int units = p.B * G_kv;
  const int s = int(blockIdx.x / unsigned(units));
  const int r = int(blockIdx.x % unsigned(units));
  const int b = r / G_kv;
  const int g_kv = r - b * G_kv;
  const int g = g_kv * p.kv_div + int(blockIdx.y);
  const int unit = b * p.G + g;             // counters and partials of the work group

  const int raw_len = p.seqlens[b];
  const int len = raw_len < 0 ? 0 : (raw_len > p.n_max ? p.n_max : raw_len);
  // Splits that hold positions (at least one, so that an empty sequence still
  // gets its zero output written).  With the merge inside this launch the
  // other splits have nothing to do; with the separate merge kernel every
  // split leaves a (possibly empty) partial.
  const int ns = p.counters == nullptr ? S : max(1, min(S, (len + p.split_len - 1) / p.split_len));
  if (s >= ns) return;
  GQA_PHASE(1);
  const int j0 = s * p.split_len;
  const int j1 = min(len, j0 + p.split_len);

  const int64_t kv_off = (int64_t(b) * G_kv + g_kv) * int64_t(p.n_max) * D;
  const uint16_t* kb = p.k + kv_off;
  const uint16_t* vb = p.v + kv_off;

  // Append (when k_new is given): the new token's k, v belong in slot
  // raw_len-1 if that slot exists.  The split holding that slot writes them
  // to the cache (the first work group of the K/V head, when several share
  // it) and into an LDS copy, which becomes the slot's row of its tile (no
  // workgroup reads that slot from the cache in this launch: the split's
  // loads end just before it).
  __shared__ __attribute__((aligned(16))) char s_new[2 * D * 2];
  const int p_new = (APPEND && raw_len >= 1 && raw_len <= p.n_max) ? raw_len - 1 : -1;
  const bool owner = APPEND && p_new >= j0 && p_new < j1;
  if (owner && threadIdx.x < 2 * C::kChunks) {
    const int c = threadIdx.x % C::kChunks;
    const bool is_v = threadIdx.x >= C::kChunks;
    const u32x4_t w = ld16((is_v ? p.v_new : p.k_new) + (int64_t(b) * G_kv + g_kv) * D + c * 8);
    if (g % p.kv_div == 0) st16(const_cast<uint16_t*>(is_v ? vb : kb) + int64_t(p_new) * D + c * 8, w);
    *reinterpret_cast<u32x4_t*>(s_new + (is_v ? D * 2 : 0) + c * 16) = w;
  }

  // Queries of the group: B operand of the score MFMA, lane = head lo of head
  // block hb, k-slot group hi covers dims 8*(4*ks + hi) .. +7.
  u32x4_t qop[NHB][C::kSteps];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hl = hb * 16 + lo;
    const bool hv = hl < p.n_rep;
    const uint16_t* qrow = p.q + (int64_t(b) * p.hm.q_heads + p.hm.q_head(g, hv ? hl : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < C::kSteps; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (hv) w = ld16(qrow + (4 * ks + hi) * 8);
      qop[hb][ks] = w;
    }
  }

  f32x4_t acc[NHB][C::kColBlocks];
  float mrun[NHB], lrun[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    mrun[hb] = -INFINITY;
    lrun[hb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb) acc[hb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = p.scale * kLog2e;
  char* myv = smem + wave * C::kWaveLds;
  char* myk = myv + kKT * C::kPitch;

  // Positions [j0, j1) through buffer resources that end at j1: loads past
  // the end return zeros without touching memory, so the loads need no
  // branches and the tile pipeline below has a fixed shape.
  const int nvalid = owner ? p_new - j0 : (j1 > j0 ? j1 - j0 : 0);
  // positions this split attends: the cached ones, plus the appended token
  const int rel_new = owner ? p_new - j0 : -1;
  const int tile_new = owner ? rel_new / kKT : -1;
  const int nattend = owner ? rel_new + 1 : nvalid;
  const uint32_t vbytes = uint32_t(nvalid) * uint32_t(D * 2);
  const __amdgpu_buffer_rsrc_t rk = rsrc(kb + int64_t(j0) * D, vbytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(vb + int64_t(j0) * D, vbytes);
  // K and V rows land 16 bytes per lane, each 64-lane load covering 64 /
  // kChunks whole rows (1 KB of contiguous cache), and go through the wave's
  // LDS area: K in the score MFMA's A layout, V for the transposing reads.
  const int row_lane = lane * 16;
  // Both streams carry the non-temporal hint (each row is read once per work
  // group; K with it measured 5-7% faster at every decode shape).  At d = 128
  // the next tile's K loads are issued as soon as this tile's K rows are in
  // LDS and its V loads once V is (1-2% faster at d = 128 than issuing both
  // after V; 2.6% slower at d = 64, which keeps the single issue point).
  constexpr bool kSplitPrefetch = D == 128;
  typedef u32x4_t KTile[C::kTileLoads];
  typedef u32x4_t VTile[C::kTileLoads];
  // (each group of loads is kept together and in program order, so that the
  // wait before a tile's use covers just the loads issued before it)
  auto load_k = [&](int tile, KTile& kr) {
    const int base = tile * (kKT * D * 2);
#pragma unroll
    for (int t = 0; t < C::kTileLoads; ++t)
      kr[t] = __builtin_amdgcn_raw_buffer_load_b128(rk, base + row_lane + t * 1024, 0, kNonTemporal);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_v = [&](int tile, VTile& vr) {
    const int base = tile * (kKT * D * 2);
#pragma unroll
    for (int t = 0; t < C::kTileLoads; ++t)
      vr[t] = __builtin_amdgcn_raw_buffer_load_b128(rv, base + row_lane + t * 1024, 0, kNonTemporal);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_tile = [&](int tile, KTile& kr, VTile& vr) {
    load_k(tile, kr);
    load_v(tile, vr);
  };

  // V^T operand of the output MFMA by transposing LDS reads: within each
  // 16-lane group (fixed hi), lanes 4e..4e+3 address row 4*hi + e (4
  // consecutive dims each) and lane lo receives dim lo of those 4 rows, i.e.
  // keys 4*hi + e (first read) and 16 + 4*hi + e (second read): exactly the
  // keys whose weights the lane holds after the score MFMA.
  const int vt_lane = (4 * hi + (lo >> 2)) * C::kPitch + (lo & 3) * 8;

  auto process = [&](int tile, KTile& kr, VTile& vr, int nv, bool prefetch) {
    // K rows of this tile into the wave's LDS area, chunk c of row r at
    // position c ^ kswz(r) (unpadded rows; the A-operand reads below then hit
    // every bank once per 16 lanes), and V rows (padded rows)
#pragma unroll
    for (int t = 0; t < C::kTileLoads; ++t) {
      const int idx = t * 64 + lane;
      const int r = idx / C::kChunks, c = idx % C::kChunks;
      *reinterpret_cast<u32x4_t*>(myk + r * (D * 2) + ((c ^ kswz<D>(r)) << 4)) = kr[t];
      if constexpr (!kSplitPrefetch) *reinterpret_cast<u32x4_t*>(myv + r * C::kPitch + c * 16) = vr[t];
    }
    if constexpr (kSplitPrefetch) {
      // K is in LDS: the next tile's K loads go out while this tile's V lands
      if (prefetch) load_k(tile + nw, kr);
#pragma unroll
      for (int t = 0; t < C::kTileLoads; ++t) {
        const int idx = t * 64 + lane;
        const int r = idx / C::kChunks, c = idx % C::kChunks;
        *reinterpret_cast<u32x4_t*>(myv + r * C::kPitch + c * 16) = vr[t];
      }
    }
    // the appended token is row rel_new of its tile: its cache row was not
    // loaded (the loads end before it), so its k, v come from the LDS copy
    if constexpr (APPEND) {
      if (tile == tile_new && lane < C::kChunks) {
        const int r = rel_new % kKT;
        *reinterpret_cast<u32x4_t*>(myk + r * (D * 2) + ((lane ^ kswz<D>(r)) << 4)) =
            *reinterpret_cast<const u32x4_t*>(s_new + lane * 16);
        *reinterpret_cast<u32x4_t*>(myv + r * C::kPitch + lane * 16) =
            *reinterpret_cast<const u32x4_t*>(s_new + D * 2 + lane * 16);
      }
    }
    // this tile's registers are free: fetch the wave's next tile into them
    if (prefetch) {
      if constexpr (kSplitPrefetch) load_v(tile + nw, vr);
      else load_tile(tile + nw, kr, vr);
    }
    lds_wave_sync();
    // scores: A = K rows 16*blk + lo, chunk 4*ks + hi, from LDS
    u32x4_t kop[2][C::kSteps];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int ks = 0; ks < C::kSteps; ++ks)
        kop[blk][ks] = *reinterpret_cast<const u32x4_t*>(myk + (16 * blk + lo) * (D * 2) +
                                                         (((4 * ks + hi) ^ kswz<D>(16 * blk + lo)) << 4));
    f32x4_t sacc[NHB][2];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::kSteps; ++ks)
          a = mfma16<DT>(kop[blk][ks], qop[hb][ks], a);
        sacc[hb][blk] = a;
      }

    // online softmax; lane holds keys 16*blk + 4*hi + r of the tile, head lo
    const int rel0 = tile * kKT + 4 * hi;
    u32x4_t pop[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float t2[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = rel0 + 16 * blk + r < nv ? sacc[hb][blk][r] * c2 : -INFINITY;
          t2[blk][r] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = max_over_rows(tmax);
      const float mn = fmaxf(mrun[hb], tmax);      // finite: the tile's first position is valid
      const float alpha = __builtin_amdgcn_exp2f(mrun[hb] - mn);
      mrun[hb] = mn;
      uint32_t w[4];
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const uint32_t pk = H16::pack2(__builtin_amdgcn_exp2f(t2[blk][2 * r2] - mn),
                                         __builtin_amdgcn_exp2f(t2[blk][2 * r2 + 1] - mn));
          w[blk * 2 + r2] = pk;
          lsum += H16::lo(pk) + H16::hi(pk);
        }
      lrun[hb] = fmaf(lrun[hb], alpha, lsum);
      pop[hb] = u32x4_t{w[0], w[1], w[2], w[3]};
#pragma unroll
      for (int cb = 0; cb < C::kColBlocks; ++cb) acc[hb][cb] *= alpha;
    }

    lds_wave_sync();
    // weighted sum of values
    const char* vt = myv + vt_lane;
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb) {
      const i16x4_t a4 = lds_read_tr16(vt + cb * 32);
      const i16x4_t b4 = lds_read_tr16(vt + 16 * C::kPitch + cb * 32);
      const u32x4_t vop = __builtin_bit_cast(u32x4_t, i16x8_t{a4[0], a4[1], a4[2], a4[3], b4[0], b4[1], b4[2], b4[3]});
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) acc[hb][cb] = mfma16<DT>(vop, pop[hb], acc[hb][cb]);
    }
  };

  // Wave w takes tiles w, w + nw, w + 2 nw, ...; each tile's processing
  // issues the loads of the next one into the registers it has just freed.
  const int ntiles = (nattend + kKT - 1) / kKT;
  // the LDS copy of k_new, v_new is read by whichever wave has the slot's
  // tile (meeting here, before the tile loads go out, measured faster than
  // after them)
  if constexpr (APPEND) {
    if (owner) __syncthreads();
  }
  KTile ka;
  VTile va;
  int tile = wave;
  load_tile(tile, ka, va);
  for (; tile < ntiles; tile += nw) {
    process(tile, ka, va, nattend, true);
    if (tile == wave) GQA_PHASE(2);
  }
  GQA_PHASE(3);

  // per-head normaliser: the four lanes of a head hold disjoint positions
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float x = lrun[hb];
    x += shfl_xor(x, 16);
    x += shfl_xor(x, 32);
    lrun[hb] = x;
  }

  // Merge the waves through LDS, one head block at a time: every wave leaves
  // its (max, normaliser) per head and its output columns; then each thread
  // combines 4 columns of one head -- recomputing that head's merged maximum
  // and per-wave factors itself, which costs a few exps but no serial step
  // and no extra barrier -- and writes the output (one split) or this
  // split's partial result.  The code after the main loop runs once per
  // workgroup, from a cold instruction cache, so it is kept short.
  float* sm_o = reinterpret_cast<float*>(smem);
  f32x2_t* sm_ml = reinterpret_cast<f32x2_t*>(sm_o + kMaxWaves * 16 * C::kMergeRow);
  constexpr int kC4 = D / 4;
  const UnitPartials<D> up(p, b, g);
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb)
      *reinterpret_cast<f32x4_t*>(sm_o + (wave * 16 + lo) * C::kMergeRow + 16 * cb + 4 * hi) = acc[hb][cb];
    if (hi == 0) sm_ml[wave * 16 + lo] = f32x2_t{mrun[hb], lrun[hb]};
    __syncthreads();
    const int nh = min(16, p.n_rep - 16 * hb);
    for (int t = threadIdx.x; t < nh * kC4; t += blockDim.x) {
      const int hl = t / kC4;
      const int c4 = t % kC4;
      f32x2_t ml[kMaxWaves];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w) {
        ml[w] = w < nw ? sm_ml[w * 16 + hl] : f32x2_t{-INFINITY, 0.f};
        if (ml[w][1] > 0.f) M = fmaxf(M, ml[w][0]);
      }
      float L = 0.f;
      f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kMaxWaves; ++w) {
        if (w < nw) {
          const float f = ml[w][1] > 0.f ? __builtin_amdgcn_exp2f(ml[w][0] - M) : 0.f;
          L = fmaf(ml[w][1], f, L);
          O += f * *reinterpret_cast<const f32x4_t*>(sm_o + (w * 16 + hl) * C::kMergeRow + c4 * 4);
        }
      }
      if (ns == 1) {
        const float inv = L > 0.f ? __builtin_amdgcn_rcpf(L) : 0.f;
        *reinterpret_cast<uint2*>(p.out + (int64_t(b) * p.hm.o_heads + p.hm.o_head(g, 16 * hb + hl)) * D + c4 * 4) =
            make_uint2(H16::pack2(O[0] * inv, O[1] * inv), H16::pack2(O[2] * inv, O[3] * inv));
      } else {
        const int pr = (16 * hb + hl) * S + s;       // within the unit's partials
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O), up.o, pr * (D * 4) + c4 * 16, 0,
                                               kDeviceCoherent);
        if (c4 == 0)
          __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(M), __float_as_uint(L)}, up.ml, pr * 8, 0,
                                                kDeviceCoherent);
      }
    }
  }
  if (ns == 1 || p.counters == nullptr) {
#ifdef GQA_DECODE_TIMELINE
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    GQA_PHASE(4);
    GQA_PHASE(6);
#endif
    return;
  }

  // Split merge by the last workgroup of this (b, g) to finish.  Each thread
  // waits until its device-coherent partial stores are acknowledged before the
  // workgroup counts itself in; the workgroup that completes the count reads
  // every partial back with device-coherent loads issued after that.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  GQA_PHASE(4);
  if (threadIdx.x == 0) {
    const int old = atomicAdd(p.counters + unit, 1);
    s_last = (old == ns - 1);
  }
  __syncthreads();
  GQA_PHASE(5);
  if (!s_last) {
    GQA_PHASE(6);
    return;
  }
  if (threadIdx.x == 0)            // ready for the next call (nothing reads it in this one)
    __hip_atomic_store(p.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int kC8 = D / 8;
  auto merge_all = [&](auto NB) {
#pragma unroll 1
    for (int t = threadIdx.x; t < p.n_rep * kC8; t += blockDim.x)
      merge_item<D, DT, decltype(NB)::value>(p, up, b, ns, g, t / kC8, t % kC8);
  };
  if (ns <= 2) merge_all(std::integral_constant<int, 2>{});
  else if (ns <= 4) merge_all(std::integral_constant<int, 4>{});
  else merge_all(std::integral_constant<int, 8>{});
#ifdef GQA_DECODE_TIMELINE
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  GQA_PHASE(6);
#endif
}

// Static LDS of the decode kernel (tiles and merge area, the appended row,
// the merge flag), and the per-workgroup total above which only one
// workgroup fits in a compute unit's 160 KB.
template <int D>
constexpr size_t kDecodeStaticLds = size_t(Cfg<D>::kLds) + 2 * D * 2 + 16;
constexpr size_t kOnePerCuLds = 82 * 1024;
constexpr int64_t kOnePerCuGrid = 1024;
static_assert(kDecodeStaticLds<128> < kOnePerCuLds, "padding");

template <int D, int NHB, int DT, bool APPEND>
hipError_t launch_t(const DecodeProblem& p, hipStream_t stream) {
  const int64_t blocks = int64_t(p.B) * (p.G / p.kv_div) * p.num_splits;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // one wave per 32-position tile of a split, at most four
  const int tiles = (p.split_len + kKT - 1) / kKT;
  const int waves = tiles >= 4 ? 4 : (tiles >= 2 ? 2 : 1);
  // A grid of several rounds of workgroups at d = 128 runs one workgroup per
  // compute unit (unused dynamic LDS makes a second one not fit): two resident
  // workgroups keep 128 KB of tiles in flight per compute unit, past the point
  // where more requests only lengthen each one's round trip (64 sequences of
  // ragged lengths up to 32768 in 11 splits, 5632 workgroups: 777 us against
  // 802 in a direct-call loop).  Grids of one or two rounds keep two per
  // compute unit (a 384-workgroup grid would take two rounds instead of one).
  const int64_t wgs = blocks * p.kv_div;
  const size_t lds_pad = (D == 128 && wgs >= kOnePerCuGrid) ? kOnePerCuLds - kDecodeStaticLds<D> : 0;
  hipLaunchKernelGGL((decode_mfma_kernel<D, NHB, DT, APPEND>), dim3(unsigned(blocks), unsigned(p.kv_div)),
                     dim3(64 * waves), lds_pad, stream, p);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_supports(int n_rep, int d, int num_splits, int split_len) {
  // Byte offsets of the buffer instructions are 32-bit: a split's K/V bytes
  // (plus the prefetch of up to 4 tiles past its end, with margin) and a unit's
  // partial results must stay below 2^31.
  const int64_t reach = (int64_t(split_len) + 16 * kKT) * d * 2;
  const int64_t partials = int64_t(n_rep) * num_splits * d * 4;
  return (d == 64 || d == 128) && n_rep >= 1 && n_rep <= 32 && reach < (int64_t(1) << 31) &&
         partials < (int64_t(1) << 31);
}

template <int DT, bool APPEND>
hipError_t launch_dt(const DecodeProblem& p, hipStream_t stream) {
  if (p.d == 128)
    return p.n_rep <= 16 ? launch_t<128, 1, DT, APPEND>(p, stream) : launch_t<128, 2, DT, APPEND>(p, stream);
  return p.n_rep <= 16 ? launch_t<64, 1, DT, APPEND>(p, stream) : launch_t<64, 2, DT, APPEND>(p, stream);
}

hipError_t launch_decode_mfma(const DecodeProblem& p, hipStream_t stream) {
  if (!abi_ok(p)) return kAbiMismatch;
  if (p.B <= 0 || p.num_splits <= 0) return hipSuccess;
  if (p.kv_div < 1 || p.G < 1 || p.G % p.kv_div != 0) return hipErrorInvalidValue;
  // the fused append is a variant of its own (the plain decode's code is unchanged by it)
  if (p.k_new != nullptr)
    return p.dtype == kF16 ? launch_dt<kF16, true>(p, stream) : launch_dt<kBF16, true>(p, stream);
  return p.dtype == kF16 ? launch_dt<kF16, false>(p, stream) : launch_dt<kBF16, false>(p, stream);
}

}  // namespace gqa
