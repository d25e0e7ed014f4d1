// Causal GQA prefill on the gfx950 matrix cores (bfloat16 or IEEE half in,
// float32 accumulate; "16-bit" below is whichever of the two the call uses).
//
// Definition: query position i of head h attends keys 0..i of K/V head
// floor(h*G/H) through softmax(scale * q.k) and a weighted sum of v (fogdragon
// CSDN blog: the context phase runs in parallel over the prompt, each position
// seeing only its past; GQA paper section 2.2 for the grouping).
//
// Work unit: one workgroup of NW waves (8 at d = 128, 4 at d = 64) per (b, g,
// head quad, query tile).  Each wave owns 32 query positions of one head; the
// waves of a workgroup cover 4 heads of one group x NW/4 consecutive
// 32-position blocks (n_rep >= 3; when n_rep is not a multiple of 4 the
// group's last quad is padded with waves that store nothing), or 2 heads x
// NW/2 blocks (n_rep = 2), or 1 head x NW blocks (n_rep = 1), so every K/V
// tile staged in LDS is used by 32*NW query rows.  Per 64-key tile and wave:
//
//   S^T[key][row] = K[key][:] . Q[row][:]        32x32x16 16-bit MFMA (2 x 8),
//                   A = K tile from LDS, B = the wave's queries (registers)
//   mask j > i on tiles that reach the diagonal; online softmax in base 2,
//   float32, one query row per lane column (max/sum in-lane plus one exchange)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row] 32x32x16 MFMA (4 x 4),
//                   A = V^T read from the row-major V tile in LDS by
//                   transposing reads, B = the 16-bit weights, already in place
//
// K/V tiles are double-buffered in LDS (layouts below) and arrive by buffer
// loads that write LDS directly, with no register staging: the next tiles'
// loads are issued at the start of an iteration into the buffers the previous
// one freed and land during its math, one barrier per tile; the weighted sum of a tile is
// deferred by one iteration so that each iteration hands the matrix unit and
// the vector unit independent work.  Softmax work per score: one FMA
// (scale folded in), one hardware exp2 (weights below 2^-126 may flush to
// zero), a third of a max3, half a 16-bit pack, half a
// 16-bit dot2 for the normaliser (which sums the rounded weights).  The
// reference maximum a row's weights are taken against moves only when a tile
// raises the row's maximum by more than kLazyLog2 (base 2): weights then stay
// below 2^kLazyLog2 and the running output is rescaled rarely (after the first
// tiles, almost never on data of moderate range).  Query tiles are issued
// heaviest first, and the query tiles of a (b, g) stay on one XCD (consecutive
// workgroups go to consecutive XCDs) so its K/V stays in that XCD's L2.

#include "device_common.h"
#include "internal.h"

#include <type_traits>

namespace gqa {
namespace {

constexpr int kKT = 64;     // keys per tile
constexpr int kQT = 32;     // query positions per wave
constexpr int kXcds = 8;
// Largest base-2 growth of a row maximum absorbed without rescaling (weights
// up to 2^8 are exact enough in 16 bits and harmless in float32 sums).
constexpr float kLazyLog2 = 8.f;


// LDS tiles, 64 banks of 4 bytes, rows unpadded and 16-byte chunks XOR-permuted
// inside each row so that the operand reads below hit all banks:
//  * K row-major: chunk c of key r sits at c ^ ksw(r).
//  * V row-major: chunk c of key k sits at c ^ vsw(k); the PV operand (V^T)
//    comes from transposing LDS reads.
// Tiles arrive by buffer loads that write LDS directly (16 bytes per lane, lane
// i at base + 16 i): each lane fetches the global chunk that belongs at its
// LDS position, so the permutation costs nothing at write time.
template <int D>
struct PCfg {
  static constexpr int kSteps = D / 16;          // QK k-steps (k = 16)
  static constexpr int kColBlocks = D / 32;      // PV output blocks of 32 dims
  static constexpr int kChunks = D / 8;          // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kKT * kRowBytes;
  static constexpr int kDma = kTileBytes / 1024; // 64-lane x 16-byte loads per tile
};
template <int D>
__device__ __forceinline__ int ksw(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vsw(int k) { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lanes 4e..4e+3 each address 4 consecutive 16-bit values of row e of
// a 4 x 16 block, and lane i receives column i of the 4 rows.
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(const_cast<char*>(p)));
}

// 32x32x16 MFMA on raw 16-bit operands: bfloat16 or IEEE half (DT).
template <int DT>
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int V> using IC = std::integral_constant<int, V>;

template <int D, int NW, int DT>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_mfma_kernel(PrefillProblem p) {
  using C = PCfg<D>;
  using H16 = Half16<DT>;
  static_assert(C::kDma % NW == 0, "tile loads split evenly over the waves");
  constexpr int kDmaW = C::kDma / NW;            // per wave per tile (K and V each)
  constexpr int kMfmaPerTile = 2 * C::kSteps + 4 * C::kColBlocks;   // scores + weighted sum
  constexpr int kValuPerMfma = 128 / kMfmaPerTile;                  // ~120 softmax instructions per tile
  // separate arrays per slot: the compiler then knows which loads in flight
  // each LDS read may depend on
  __shared__ __attribute__((aligned(16))) char sk0[C::kTileBytes];
  __shared__ __attribute__((aligned(16))) char sk1[C::kTileBytes];
  __shared__ __attribute__((aligned(16))) char sv0[C::kTileBytes];
  __shared__ __attribute__((aligned(16))) char sv1[C::kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  const int nre = p.n_rep <= 2 ? p.n_rep : 4;     // head slots per workgroup
  const int tb_per_wg = NW / nre;                  // 32-position blocks per workgroup
  const int n_hq = (p.n_rep + nre - 1) / nre;      // (the last quad may be padded)
  const int rows_wg = kQT * tb_per_wg;
  const int n_qt = (p.T + rows_wg - 1) / rows_wg;
  const int units = p.B * p.G * n_hq;
  int unit, qt_rank;
  if (units % kXcds == 0) {
    // keep a unit's query tiles on one XCD: workgroup i runs on XCD i % 8
    const int x = int(blockIdx.x % kXcds);
    const int i = int(blockIdx.x / kXcds);
    const int per_xcd = units / kXcds;
    unit = x * per_xcd + i % per_xcd;
    qt_rank = i / per_xcd;
  } else {
    unit = int(blockIdx.x % unsigned(units));
    qt_rank = int(blockIdx.x / unsigned(units));
  }
  const int qt = n_qt - 1 - qt_rank;              // heaviest first
  const int hq = unit % n_hq;
  const int g = (unit / n_hq) % p.G;
  const int b = unit / (n_hq * p.G);

  const int qr = hq * nre + (wave % nre);          // query of the group this wave owns
  // A padding slot of the last quad (qr >= n_rep) computes on a copy of the
  // group's last query and stores nothing: the workgroup's tile loads and
  // barriers stay the same for every wave.
  const bool q_valid = qr < p.n_rep;
  const int t_base = qt * rows_wg + (wave / nre) * kQT;
  const int t_row = t_base + l32;                  // this lane's query row
  const int t_last = min(p.T, (qt + 1) * rows_wg) - 1;
  // Row t sits at position ctx + t and sees positions 0 .. min(ctx + t, kv_cap - 1).
  const int ctx = p.ctx_lens ? max(p.ctx_lens[b], 0) : 0;
  const int last_pos = p.kv_cap - 1;
  const int a_row = min(ctx + t_row, last_pos);            // this lane's last visible position
  const int a_wave = min(ctx + t_base + kQT - 1, last_pos); // ... of the wave's last row
  const int kv_end = min(ctx + t_last, last_pos) + 1;       // positions any row here sees
  const int n_kt = (kv_end + kKT - 1) / kKT;

  const int64_t kv_row = p.kv_pstride;               // elements between positions
  const uint16_t* kbase = p.k + int64_t(b) * p.kv_bstride + int64_t(g) * p.kv_gstride;
  const uint16_t* vbase = p.v + int64_t(b) * p.kv_bstride + int64_t(g) * p.kv_gstride;
  // Positions [0, kv_end) of this (b, g) through buffer resources that end
  // there: loads past the end write zeros to LDS without a memory access, so
  // the tile loads need no per-lane branches.  (The host keeps every offset
  // below 2^31.)
  const int row_bytes = int(kv_row) * 2;
  const uint32_t kv_bytes = uint32_t((kv_end - 1) * row_bytes + D * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase), 0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase), 0, kv_bytes, 0x00020000);
  // this lane's source offsets within a tile: LDS chunk position s of row r
  // holds global chunk s ^ swizzle(r)
  int koff[kDmaW], voff[kDmaW];
#pragma unroll
  for (int i = 0; i < kDmaW; ++i) {
    const int pos = (wave * kDmaW + i) * 64 + lane;
    const int r = pos / C::kChunks, s = pos % C::kChunks;
    koff[i] = r * row_bytes + ((s ^ ksw<D>(r)) << 4);
    voff[i] = r * row_bytes + ((s ^ vsw<D>(r)) << 4);
  }
  auto tile_load = [&](__amdgpu_buffer_rsrc_t rs, const int* off, int kt, char* dst) {
    const int base = kt * kKT * row_bytes;
#pragma unroll
    for (int i = 0; i < kDmaW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + (wave * kDmaW + i) * 1024), 16,
          base + off[i], 0, 0, 0);
  };
  auto kslot = [&](auto P) -> char* {
    if constexpr (decltype(P)::value == 0) return sk0; else return sk1;
  };
  auto vslot = [&](auto P) -> char* {
    if constexpr (decltype(P)::value == 0) return sv0; else return sv1;
  };

  // queries: B operand, lane column = row l32, k-slot group h2 -> dims 16*ks + 8*h2 .. +7.
  // A negative scale is folded into the queries (exact sign flip).
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;
  // (a zero scale is replaced by a tiny one: the weights are then exactly
  // uniform, and masked scores still map to exactly zero weight)
  const float c2 = p.scale == 0.f ? 1e-30f : fabsf(p.scale) * kLog2e;
  u32x4_t qop[C::kSteps];
  {
    const bool rvq = t_row < p.T;
    const uint16_t* qrow = p.q + ((int64_t(b) * p.T + (rvq ? t_row : 0)) * p.hm.q_heads +
                                  p.hm.q_head(g, q_valid ? qr : p.n_rep - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < C::kSteps; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (rvq) w = ld16(qrow + 16 * ks + 8 * h2);
      w ^= u32x4_t{qsign, qsign, qsign, qsign};
      qop[ks] = w;
    }
  }

  f32x16_t acc[C::kColBlocks];
#pragma unroll
  for (int cb = 0; cb < C::kColBlocks; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  float mrun = -INFINITY;     // running max of the raw scores of this lane's row
  float lrun = 0.f;           // this lane's share of the normaliser

  // scores of one tile: lane holds S^T[key0 + 32*kb + 8*(r/4) + 4*h2 + r%4][t_row];
  // two independent accumulator chains (key blocks kb = 0, 1) interleaved.
  // K operand: row l32 (+32), chunk 2 ks + h2, permuted: byte offset
  // (32 ks + 16 h2) ^ 16 ksw(l32) = kx ^ 32 ks inside the row.
  const int kx = l32 * C::kRowBytes + ((h2 ^ ksw<D>(l32)) << 4);
  auto qk = [&](const char* sk, f32x16_t* sc) {
    const f32x16_t zero = {};
#pragma unroll
    for (int ks = 0; ks < C::kSteps; ++ks) {
      const char* a = sk + (kx ^ (32 * ks));
      const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(a);
      const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(a + 32 * C::kRowBytes);
      sc[0] = mfma32<DT>(k0, qop[ks], ks == 0 ? zero : sc[0]);
      sc[1] = mfma32<DT>(k1, qop[ks], ks == 0 ? zero : sc[1]);
    }
  };

  // Online softmax of one tile's scores (masked near the diagonal): 16-bit
  // weights as PV B operands (one per 16-key step u: keys 16u + 8*(e/4) +
  // 4*h2 + e%4), the new running maximum, and the factor the running output
  // must be scaled by before these weights are added to it.
  auto softmax = [&](f32x16_t* sc, int key0, bool masked, u32x4_t* pop, float& alpha, bool& rescale) {
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (key > a_row) sc[kb][r] = -INFINITY;
        }
    }
    float tmax = mrun;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = fmaxf(fmaxf(tmax, sc[kb][r]), sc[kb][r + 1]);
    // row maximum over both lane halves (one register swap, no LDS round trip);
    // finite: key 0 precedes every row
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                     false, false);
    const float mn = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const bool grow = __any(mrun == -INFINITY || (mn - mrun) * c2 > kLazyLog2);
    const float mref = grow ? mn : mrun;            // wave-uniform choice
    const float mc = mref * c2;
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int r0 = 8 * (u & 1) + 2 * e2;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[u >> 1][r0], c2, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[u >> 1][r0 + 1], c2, -mc));
        w[e2] = H16::pack2(p0, p1);
        lsum = H16::sum2(w[e2], lsum);
      }
      pop[u] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    alpha = grow ? (mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun * c2 - mc)) : 1.f;
    rescale = grow;
    lrun = fmaf(lrun, alpha, lsum);
    mrun = mref;
  };

  // O^T += V^T P^T.  A operand for k-step u, lane (l32, h2): V[key][32 cb +
  // l32] for keys 16u + 8*(e/4) + 4*h2 + e%4, e = 0..7 -- two transposing
  // reads of 4 keys each.  In the read, lane l32 % 16 = 4 e4 + j4 addresses key
  // 4 h2 + e4 (+16u, +8) at dims 32 cb + 16 (l32 / 16) + 4 j4, a permuted byte
  // offset of vx ^ 64 cb.
  const int e4 = (l32 >> 2) & 3, j4 = l32 & 3;
  const int vx = (4 * h2 + e4) * C::kRowBytes +
                 (64 * (D == 128 ? e4 : (e4 >> 1)) + 32 * (l32 >> 4) + 8 * j4);
  auto pv = [&](const u32x4_t* pop, const char* sv) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4_t vop[C::kColBlocks];
#pragma unroll
      for (int cb = 0; cb < C::kColBlocks; ++cb) {
        const char* a = sv + (vx ^ (64 * cb)) + 16 * u * C::kRowBytes;
        const i16x4_t lo = lds_read_tr16(a);
        const i16x4_t hi = lds_read_tr16(a + 8 * C::kRowBytes);
        vop[cb] = __builtin_bit_cast(u32x4_t, i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
#pragma unroll
      for (int cb = 0; cb < C::kColBlocks; ++cb) acc[cb] = mfma32<DT>(vop[cb], pop[u], acc[cb]);
    }
  };
  auto rescale_acc = [&](float alpha) {
    asm volatile("");       // keeps the (rare) rescale a branch rather than a multiply by 1
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb) acc[cb] *= alpha;
  };
  // every wave's tile loads have landed, then all waves meet
  auto tile_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // Software pipeline over key tiles.  Iteration t issues, as one scheduling
  // region with no branch inside: the score MFMAs of tile t+1, the weighted
  // sum of tile t-1 (its weights were made one iteration earlier) and the
  // softmax of tile t -- independent work for the matrix and the vector unit
  // of the same wave.  When tile t moved a row's reference maximum (rare),
  // the running output -- which by then holds the tiles up to t-1 -- is
  // rescaled at the end of the iteration, before tile t's weights are added
  // at the next one.  LDS: K slot (t+1)&1 holds K(t+1), V slot (t+1)&1 holds
  // V(t-1); the loads of K(t+2) and V(t) go, at the start of the iteration,
  // to the slots t&1 the previous iteration freed, and land during it.  Tiles
  // before t_split lie wholly below every row of the workgroup (no mask) and
  // have a successor; the rest take the masked path.  The slot parity P = t&1
  // is a compile-time constant at every call site.
  const int t_split = min(n_kt - 1, min(ctx + qt * rows_wg, last_pos) / kKT);
  tile_load(rk, koff, 0, sk0);
  tile_load(rk, koff, 1, sk1);     // (reads as zeros past the end)
  tile_barrier();
  // Two score buffers alternate between "this tile" and "next tile" (the
  // loops below are unrolled by two), so no copy sits between a tile's score
  // MFMAs and its softmax.
  f32x16_t sa[2], sb[2];
  qk(sk0, sa);
  // every wave has read K(0) before the first iteration overwrites its slot
  __syncthreads();
  u32x4_t pprev[4];
  float alpha_prev = 1.f;
  bool rescale_prev = false;

  // one unmasked iteration (with_pv is a constant at each call site, so the
  // region below has no branch); cur holds tile t's scores, nxt receives t+1's
  auto iter_unmasked = [&](int t, auto P, bool with_pv, f32x16_t* cur, f32x16_t* nxt) {
    constexpr int Q = 1 - decltype(P)::value;
    tile_load(rk, koff, min(t + 2, n_kt - 1), kslot(P));
    tile_load(rv, voff, t, vslot(P));
    qk(kslot(IC<Q>{}), nxt);
    if (with_pv) pv(pprev, vslot(IC<Q>{}));
    softmax(cur, t * kKT, false, pprev, alpha_prev, rescale_prev);
    // Issue order for the region above at d = 128: the tile loads, 8 operand
    // reads, then each MFMA followed by a share of the softmax's vector
    // instructions and the next operand read (left to itself the compiler
    // puts all MFMAs first and the softmax after them; this order measured
    // ~2% faster at d = 128 and ~1% slower at d = 64, which keeps the
    // compiler's order).
    if constexpr (D == 128) {
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * kDmaW, 0);    // tile loads
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);            // LDS reads
#pragma unroll
      for (int i = 0; i < kMfmaPerTile; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // vector ALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // LDS read
      }
    }
    // the weights are made here, ahead of the branch (not sunk into the next
    // iteration, which would leave the matrix work above without vector work)
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(pprev[u]));
    if (rescale_prev) rescale_acc(alpha_prev);
    tile_barrier();
  };
  // one iteration on a tile that may reach the diagonal
  auto iter_masked = [&](int t, auto P, f32x16_t* cur, f32x16_t* nxt) {
    constexpr int Q = 1 - decltype(P)::value;
    if (t + 2 < n_kt) tile_load(rk, koff, t + 2, kslot(P));
    tile_load(rv, voff, t, vslot(P));
    const bool next_active = t + 1 < n_kt && (t + 1) * kKT <= a_wave;
    if (next_active) qk(kslot(IC<Q>{}), nxt);
    if (t > 0 && (t - 1) * kKT <= a_wave) pv(pprev, vslot(IC<Q>{}));
    if (t * kKT <= a_wave) {
      softmax(cur, t * kKT, true, pprev, alpha_prev, rescale_prev);
    } else {
      rescale_prev = false;
    }
    if (rescale_prev) rescale_acc(alpha_prev);
    tile_barrier();
  };
  // tile t's scores are in sa for even t, in sb for odd t
  int t = 0;
  if (t_split > 0) {
    iter_unmasked(0, IC<0>{}, false, sa, sb);
    for (t = 1; t + 1 < t_split; t += 2) {
      iter_unmasked(t, IC<1>{}, true, sb, sa);
      iter_unmasked(t + 1, IC<0>{}, true, sa, sb);
    }
    if (t < t_split) {
      iter_unmasked(t, IC<1>{}, true, sb, sa);
      ++t;
    }
  }
  if (t < n_kt && (t & 1)) {
    iter_masked(t, IC<1>{}, sb, sa);
    ++t;
  }
  for (; t < n_kt; t += 2) {                       // tiles that reach the diagonal
    iter_masked(t, IC<0>{}, sa, sb);
    if (t + 1 < n_kt) iter_masked(t + 1, IC<1>{}, sb, sa);
  }
  // the last tile's weighted sum (any rescale it needs was applied above)
  if ((n_kt - 1) * kKT <= a_wave) pv(pprev, ((n_kt - 1) & 1) ? sv1 : sv0);

  const float l = lrun + shfl_xor(lrun, 32);
  if (t_row < p.T && q_valid) {
    const float inv = 1.f / l;
    uint16_t* orow = p.out + ((int64_t(b) * p.T + t_row) * p.hm.o_heads + p.hm.o_head(g, qr)) * D;
#pragma unroll
    for (int cb = 0; cb < C::kColBlocks; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = 32 * cb + 8 * r4 + 4 * h2;
        const uint32_t w0 = H16::pack2(acc[cb][4 * r4] * inv, acc[cb][4 * r4 + 1] * inv);
        const uint32_t w1 = H16::pack2(acc[cb][4 * r4 + 2] * inv, acc[cb][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + col) = make_uint2(w0, w1);
      }
  }
}

}  // namespace

bool prefill_mfma_supports(int n_rep, int d, int kv_cap, int64_t kv_pstride) {
  // byte offsets of the K/V buffer loads (up to a tile past the end) stay below 2^31
  const int64_t reach = (int64_t(kv_cap) + 2 * kKT) * kv_pstride * 2;
  return (d == 64 || d == 128) && n_rep >= 1 &&
         reach < (int64_t(1) << 31);
}

template <int D, int NW>
hipError_t launch_d(const PrefillProblem& p, hipStream_t stream) {
  const int nre = p.n_rep <= 2 ? p.n_rep : 4;
  const int rows_wg = kQT * (NW / nre);
  const int64_t n_qt = (p.T + rows_wg - 1) / rows_wg;
  const int64_t blocks = n_qt * p.B * p.G * ((p.n_rep + nre - 1) / nre);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid = dim3(unsigned(blocks)), block = dim3(64 * NW);
  if (p.dtype == kF16)
    hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, kF16>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, kBF16>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillProblem& p, hipStream_t stream) {
  if (!abi_ok(p)) return kAbiMismatch;
  // d = 128: 8 waves (one workgroup per CU, by registers).  d = 64: 4 waves,
  // two workgroups per CU -- one's start and end overlap the other's tiles
  // (measured 3% faster than 8 waves at d = 64; at d = 128, 4 waves spill).
  if (p.d == 128) return launch_d<128, 8>(p, stream);
  return launch_d<64, 4>(p, stream);
}

}  // namespace gqa
