// Batch-1 fused decode-GEMV for the 3-bit format (C=12, P=4, K=16).
//
// As in the 4-bit kernel, each block's weights are never formed: SeedLM fetches
// the block's seed and coefficients and uses the rebuilt weights at once
// (paperhub.cn rebuttal text before Eq. (1); blocks of C weights = 2^e U(s) t,
// atlas.scime.ai "Approach").  The block's contribution to its row is
//   2^(e-15) sum_j t_j D_j,   D_j = sum_{i<12} x_i (z_{12j+i} - 2^15),
// and with the 16-bit Fibonacci LFSR every state is a 16-bit window of one bit
// stream b (b[0..15] = seed bits), so
//   D_j = sum_{m<27} b[12j+m] c_m - 2^15 sum_i x_i,
//   c_m = sum_{i+k=m, i<12, k<16} x_i 2^k.
// Column j's 27 bits split into bytes at bit offsets 12j, 12j+8, 12j+16 and the
// three bits at 12j+24, so D_j = H0[.] + H1[.] + H2[.] + H3[.] with
//   Hq[v] = sum_{k<8} bit_k(v) c_{8q+k}   (H3: bits 0..2 only; H0 also carries
//                                          -2^15 sum_i x_i).
// Even columns start on the stream's byte grid (bytes S0..S6 of the 63-bit
// stream), odd columns on the grid shifted by four bits (S'_q = bits 8q+4 ..
// 8q+11); column j's last byte is column j+2's first, so 16 lookups read 14
// distinct bytes.  The stream bits past the seed come from GF(2) byte tables,
// ext(s) = T0[s & 255] ^ T1[s >> 8] (64-bit entries, kept as lo/hi words).
//
// The tables depend on x, so they are built per column unit: one packed panel
// of 16 blocks = 192 columns, whose rows are 64 contiguous bytes of words, so
// a unit's loads fetch only its own bytes.  LDS rows are indexed by a stream
// byte (256 B per row):
//   region 0 row v = [H0 | H1 | H2 | H3]          (16 slots each)
//   region 1 row v = [T0lo | T1lo | T0hi | T1hi]  (16 copies each)
// One v_perm_b32 turns a byte and a per-lane constant into an address.
//
// Lane mapping: lane = 4*rho + g; the lane owns row r0+rho and slot group g of
// the unit (slots 4g..4g+3) and reads the group's four words with one 16-byte
// load and their exponent nibbles with one 2-byte load.  A half-wave thus holds
// 8 rows over 16 slots: if all its lanes read one 16-column table, two lanes
// share every bank.  Instead the lanes are split by pi = bit 2 of rho, and the
// lookups are issued in pairs of tables whose columns lie in opposite bank
// halves (H0/H1, H2/H3, T0/T1: column c and c ^ 16).  In the first read of a
// pair, pi = 0 lanes read table X at byte K_X and pi = 1 lanes table Y at byte
// K_Y; in the second read, the other way round.  The per-lane selector of the
// v_perm picks the byte and the per-lane constant the column.  Both reads of a
// pair enter the same column sum (or the same XOR for T), so no lane needs to
// know which came first, and every read covers 32 distinct banks.  The row's
// partial sum is reduced over its 4 lanes with DPP and written per unit;
// reduce_panels_kernel adds the units in a fixed order (deterministic).
#include "lfsr_device.h"
#include "lut_common.h"

namespace seedlm {
namespace {

constexpr int kThreads = 1024;  // 16 waves: 4 per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kSlots = 16;                       // blocks per column unit
constexpr int kUnitCols = 12 * kSlots;           // 192 columns
constexpr int kRowsPerSlab = 16;                 // rows per wave step

struct Smem {
  uint32_t R0[256][64];  // [H0 | H1 | H2 | H3]
  uint32_t R1[256][64];  // [T0lo | T1lo | T0hi | T1hi]
  float xs[kUnitCols];
  uint32_t gf2lo[512], gf2hi[512];  // T0 then T1, staged before replication
  int next_slab;                    // slab counter of the current segment
};
constexpr int kH0 = 0, kH1 = 16, kH2 = 32, kH3 = 48;      // region 0 columns
constexpr int kT0lo = 0, kT1lo = 16, kT0hi = 32, kT1hi = 48;  // region 1 columns
constexpr uint32_t kRegion1 = 65536;
// H2/H3 sit 32 columns after H0/H1, and T0hi/T1hi 32 after T0lo/T1lo: the
// second table pair of a region is read at this instruction offset.
constexpr uint32_t kOffHi = 4 * (kH2 - kH0);
static_assert(kH2 - kH0 == kH3 - kH1 && kT0hi - kT0lo == kT1hi - kT1lo &&
              kT0hi - kT0lo == kH2 - kH0, "pairs must share their offsets");

// v_perm selector of lut_addr<K>: address bytes [lanec.b0, src.byte K, lanec.b2, 0].
__host__ __device__ constexpr uint32_t byte_sel(int K) { return 0x0C020000u | ((4u + K) << 8); }

// Cost model of the work split: a unit's table build costs about as much as
// kBuildCost slabs of 16 rows.
constexpr int64_t kBuildCost = 40;

// Rows 8*vg .. 8*vg+7 of one table pair of a slot: the first table prices bits
// MA .. MA+7 of a byte (c_MA ..), the second bits MB .. MB+NB-1; the first also
// carries `base` (-2^15 sum x for H0).  Indices are compile-time, so c stays in
// registers.
template <int MA, int MB, int NB>
__device__ inline void build_pair(const float (&c)[27], float base, int vg, uint32_t* ta,
                                  uint32_t* tb) {
  float Ba = base, Bb = 0.f;
#pragma unroll
  for (int k = 3; k < 8; ++k) {
    if ((vg >> (k - 3)) & 1) {
      Ba += c[MA + k];
      if (k < NB) Bb += c[MB + k];
    }
  }
  float La[8], Lb[8];
  La[0] = Lb[0] = 0.f;
#pragma unroll
  for (int n = 1; n < 8; ++n) {
    const int low = __builtin_ctz(n), rest = n & (n - 1);
    La[n] = La[rest] + c[MA + low];
    Lb[n] = low < NB ? Lb[rest] + c[MB + low] : Lb[rest];
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int v = 8 * vg + n;
    ta[v * 64] = __float_as_uint(La[n] + Ba);
    tb[v * 64] = __float_as_uint(Lb[n] + Bb);
  }
}

__device__ void build_unit_lut(Smem& sm, float xval) {
  // xval: this thread's x value of the unit (threads 0..191), loaded ahead.
  const int tid = threadIdx.x;
  if (tid < kUnitCols) sm.xs[tid] = xval;
  __syncthreads();
  // Thread -> (table pair, slot, 8-row group): threads 0..511 write H0 and H2,
  // 512..1023 H1 and H3 (a choice uniform over each wave), rows 8*vg .. 8*vg+7.
  const int slot = tid & 15, vg = (tid >> 4) & 31, pair = tid >> 9;
  float xv[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) xv[i] = sm.xs[slot * 12 + i];
  // c_m: doubling upwards for m <= 14, halving downwards for m = 26..15.
  float c[27];
  c[0] = xv[0];
#pragma unroll
  for (int m = 1; m < 15; ++m) c[m] = m < 12 ? fmaf(2.f, c[m - 1], xv[m]) : 2.f * c[m - 1];
  c[26] = 32768.f * xv[11];
#pragma unroll
  for (int m = 25; m >= 15; --m) c[m] = fmaf(0.5f, c[m + 1], 32768.f * xv[m - 15]);
  if (pair == 0) {
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < 12; ++i) S += xv[i];
    build_pair<0, 16, 8>(c, -32768.f * S, vg, &sm.R0[0][kH0 + slot], &sm.R0[0][kH2 + slot]);
  } else {
    build_pair<8, 24, 3>(c, 0.f, vg, &sm.R0[0][kH1 + slot], &sm.R0[0][kH3 + slot]);
  }
}

template <typename XT>
__global__ void __launch_bounds__(kThreads, 1) gemv_lut12_kernel(const LutGroup grp) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rho = lane >> 2, g = lane & 3;
  const uint8_t* lds = reinterpret_cast<const uint8_t*>(&sm);

  const int64_t begin = grp.bounds[blockIdx.x];
  const int64_t end = grp.bounds[blockIdx.x + 1];
  // Where `begin` lies: matrix mi, column unit u, first slab sa.  This is the
  // only division of the loop; each later segment starts at the next unit.
  int mi = 0;
  while (mi + 1 < grp.n && begin >= grp.m[mi + 1].item_begin) ++mi;
  int u = 0, sa = 0;
  if (begin < end) {
    const uint32_t local = (uint32_t)(begin - grp.m[mi].item_begin);
    const uint32_t slabs = (uint32_t)grp.m[mi].slabs;
    u = (int)(local / slabs);
    sa = (int)(local - (uint32_t)u * slabs);
  }
  // The x of a segment's unit is loaded one segment ahead (threads 0..191 hold
  // one raw value each) with a buffer load whose out-of-range offset reads
  // zero: columns past the matrix enter the tables as x = 0.
  auto fetch_x = [&](int m2, int u2, bool valid) -> uint32_t {
    const LutMatrix& N = grp.m[m2];
    const int64_t c = (int64_t)u2 * kUnitCols + tid;
    const uint32_t off = (valid && tid < kUnitCols && c < N.cols)
                             ? (uint32_t)c * sizeof(XT) : 0x80000000u;
    const uint64_t xp = (uint64_t)N.x;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)xp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(xp >> 32));
    const int nbytes = __builtin_amdgcn_readfirstlane((int)(N.cols * sizeof(XT)));
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(((uint64_t)hi << 32) | lo), 0, nbytes, 0x00020000);
    if constexpr (sizeof(XT) == 2)
      return __builtin_amdgcn_raw_buffer_load_b16(xr, off, 0, 0);
    else
      return __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
  };
  auto x_value = [](uint32_t raw) -> float {
    if constexpr (sizeof(XT) == 2)
      return __half2float(__ushort_as_half((unsigned short)raw));
    else
      return __uint_as_float(raw);
  };
  uint32_t x_next = fetch_x(mi, u, begin < end);

  // GF(2) tables (built once per launch), 16 copies of each word: staged, then
  // replicated with 16-byte writes.
  if (tid < 512) {
    const uint32_t u = tid & 255;
    const uint64_t e = ext_bits<uint64_t>(tid < 256 ? u : u << 8);
    sm.gf2lo[tid] = (uint32_t)e;
    sm.gf2hi[tid] = (uint32_t)(e >> 32);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4096 / kThreads; ++k) {
    const int e = tid + k * kThreads;
    const int table = e >> 10, u = (e >> 2) & 255, part = e & 3;  // T0lo, T1lo, T0hi, T1hi
    const int src = (table & 1) * 256 + u;
    const uint32_t val = table < 2 ? sm.gf2lo[src] : sm.gf2hi[src];
    reinterpret_cast<uint4*>(&sm.R1[u][16 * table])[part] = make_uint4(val, val, val, val);
  }

  // Slots of this lane's four words: slot_j = 4g + ((j + row) & 3); slabs start
  // at multiples of 16 rows, so row & 3 == rho & 3.  First read of a pair:
  // column of H0 (pi = 0) or H1 (pi = 1), second read: the other one; region 1
  // holds the T tables in the same column pattern.
  const uint32_t pi = (rho >> 2) & 1;
  uint32_t lcA[4], lcB[4], lcTA[4], lcTB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t slot = 4u * g + ((j + rho) & 3);
    lcA[j] = 4u * (slot + 16u * pi);
    lcB[j] = 4u * (slot + 16u * (pi ^ 1u));
    lcTA[j] = lcA[j] | kRegion1;
    lcTB[j] = lcB[j] | kRegion1;
  }
  // Selectors for byte pairs (K, K+1): first read takes byte K on pi = 0 lanes
  // and K+1 on pi = 1 lanes, the second read the other way round.
  uint32_t selA[3], selB[3];
#pragma unroll
  for (int K = 0; K < 3; ++K) {
    selA[K] = pi ? byte_sel(K + 1) : byte_sel(K);
    selB[K] = pi ? byte_sel(K) : byte_sel(K + 1);
  }

  for (int64_t it = begin; it < end;) {
    const LutMatrix& M = grp.m[mi];
    const int64_t Mp = M.Mp;
    const int slabs = M.slabs;
    const int64_t ustart = M.item_begin + (int64_t)u * slabs;  // u: panel u
    const int64_t seg_end = ustart + slabs < end ? ustart + slabs : end;
    const int sb = (int)(seg_end - ustart);
    int mn = mi, un = u + 1;  // the next segment's unit
    if (un == M.np) {
      un = 0;
      ++mn;
    }
    const int64_t p = u;   // a unit is one whole 16-block panel
    const int grp4 = g;    // this lane's slot group in the panel
    const int Wp = (int)panel_stored_width(p, M.nb, kSlots);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)M.words, 0, (int)M.words_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t prsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)M.partial, 0, (int)(M.np * Mp * 4), 0x00020000);
    // Lanes outside the panel's stored width read zero words (t = 0: no
    // contribution); rows at or past Mp in the last slab read words of no row
    // of this unit (or zeros past the buffer) and store nothing.
    const bool gvalid = 4 * grp4 < Wp;
    const uint32_t wbase = gvalid ? (uint32_t)(p * Mp * kSlots + rho * Wp + 4 * grp4) * 4u
                                  : 0x80000000u;
    const uint32_t ebase =
        gvalid ? M.exp_off + (uint32_t)(p * Mp * (kSlots / 4) + rho * (Wp / 4) + grp4) * 2u
               : 0x80000000u;
    const uint32_t wstride = (uint32_t)kRowsPerSlab * (uint32_t)Wp * 4u;
    const uint32_t estride = (uint32_t)kRowsPerSlab * (uint32_t)(Wp / 4) * 2u;
    struct Slab {
      v4u w;
      uint32_t e;
    };
    // Slabs past the segment (the look-ahead of its last loads) get an
    // out-of-range offset: they read zeros and fetch nothing from memory.
    auto load = [&](int sl) {
      Slab s;
      const bool in = sl < sb;
      s.w = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc, in ? wbase + (uint32_t)sl * wstride : 0x80000000u, 0, 0);
      s.e = __builtin_amdgcn_raw_buffer_load_b16(
          rsrc, in ? ebase + (uint32_t)sl * estride : 0x80000000u, 0, 0);
      return s;
    };
    const int s_first = sa + wave;
    Slab A[2] = {load(s_first), load(s_first + kWaves)};
    const uint32_t x_this = x_next;
    x_next = fetch_x(mn < grp.n ? mn : mi, un, seg_end < end);
    __syncthreads();  // previous unit's tables and slab counter no longer in use
    if (tid == 0) sm.next_slab = sa + 2 * kWaves;
    build_unit_lut(sm, x_value(x_this));
    __syncthreads();

    auto run = [&](const Slab& q, int sl) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = q.w[k];
      // Pair read of tables (X, X+16 columns) at bytes (K, K+1) of src: the two
      // values, in either order; off = 0 for H0/H1 (T0lo/T1lo), kOffHi for
      // H2/H3 (T0hi/T1hi).
      auto pair_addr = [&](uint32_t src, uint32_t lca, uint32_t lcb, int K, uint32_t& aa,
                           uint32_t& ab) {
        aa = __builtin_amdgcn_perm(src, lca, selA[K]);
        ab = __builtin_amdgcn_perm(src, lcb, selB[K]);
      };
      // Stage 1: the GF(2) halves and H0[S0] + H1[S1], all from seed bytes 0, 1.
      uint32_t t0[4], t1[4], t2[4], t3[4];
      float hs[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t ta, tb;
        pair_addr(w[k], lcTA[k], lcTB[k], 0, ta, tb);
        t0[k] = lds_at<uint32_t>(lds, ta);
        t1[k] = lds_at<uint32_t>(lds, tb);
        t2[k] = lds_at<uint32_t>(lds, ta + kOffHi);
        t3[k] = lds_at<uint32_t>(lds, tb + kOffHi);
      }
      float ha[4], hb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t aa, ab;
        pair_addr(w[k], lcA[k], lcB[k], 0, aa, ab);
        ha[k] = lds_at<float>(lds, aa);
        hb[k] = lds_at<float>(lds, ab);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) hs[k] = ha[k] + hb[k];
      float acc = 0.f;
      // Stages 2 and 3 in two halves of two words (register pressure).
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float h[2][14];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int k = 2 * hh + kk;
          const uint32_t elo = t0[k] ^ t1[k], ehi = t2[k] ^ t3[k];
          const uint32_t lo = __builtin_amdgcn_perm(elo, w[k], 0x05040100u);   // bits 0..31
          const uint32_t hi = __builtin_amdgcn_perm(ehi, elo, 0x05040302u);    // bits 32..63
          const uint32_t lo4 = __builtin_amdgcn_alignbit(hi, lo, 4);           // bits 4..35
          const uint32_t hi4 = hi >> 4;                                        // bits 36..
          const uint32_t c2 = __builtin_amdgcn_alignbit(hi, lo, 24);           // S3, S4, ..
          const uint32_t c1 = __builtin_amdgcn_alignbit(hi4, lo4, 24);         // S'3, S'4, ..
          uint32_t aa, ab;
          // column 0: H2[S2] + H3[S3]
          pair_addr(lo, lcA[k], lcB[k], 2, aa, ab);
          h[kk][0] = lds_at<float>(lds, aa + kOffHi);
          h[kk][1] = lds_at<float>(lds, ab + kOffHi);
          // column 1: H0[S'1] + H1[S'2], H2[S'3] + H3[S'4]
          pair_addr(lo4, lcA[k], lcB[k], 1, aa, ab);
          h[kk][2] = lds_at<float>(lds, aa);
          h[kk][3] = lds_at<float>(lds, ab);
          pair_addr(c1, lcA[k], lcB[k], 0, aa, ab);
          h[kk][4] = lds_at<float>(lds, aa + kOffHi);
          h[kk][5] = lds_at<float>(lds, ab + kOffHi);
          // column 2: H0[S3] + H1[S4], H2[S5] + H3[S6]
          pair_addr(c2, lcA[k], lcB[k], 0, aa, ab);
          h[kk][6] = lds_at<float>(lds, aa);
          h[kk][7] = lds_at<float>(lds, ab);
          pair_addr(hi, lcA[k], lcB[k], 1, aa, ab);
          h[kk][8] = lds_at<float>(lds, aa + kOffHi);
          h[kk][9] = lds_at<float>(lds, ab + kOffHi);
          // column 3: H0[S'4] + H1[S'5], H2[S'6] + H3[S'7]
          pair_addr(hi4, lcA[k], lcB[k], 0, aa, ab);
          h[kk][10] = lds_at<float>(lds, aa);
          h[kk][11] = lds_at<float>(lds, ab);
          pair_addr(hi4, lcA[k], lcB[k], 2, aa, ab);
          h[kk][12] = lds_at<float>(lds, aa + kOffHi);
          h[kk][13] = lds_at<float>(lds, ab + kOffHi);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int k = 2 * hh + kk;
          const float D0 = hs[k] + (h[kk][0] + h[kk][1]);
          const float D1 = (h[kk][2] + h[kk][3]) + (h[kk][4] + h[kk][5]);
          const float D2 = (h[kk][6] + h[kk][7]) + (h[kk][8] + h[kk][9]);
          const float D3 = (h[kk][10] + h[kk][11]) + (h[kk][12] + h[kk][13]);
          const uint32_t wk = w[k];
          // t_j/16 from the coefficient nibbles (v_cvt_off_f32_i4: signed
          // nibble -> nibble/16; nibbles 0 and 2 through a byte select);
          // the 1/16 is undone by the panel reduction's scale.
          float V = __builtin_amdgcn_cvt_off_f32_i4(wk >> 16) * D0;
          V = fmaf(__builtin_amdgcn_cvt_off_f32_i4(wk >> 20), D1, V);
          V = fmaf(__builtin_amdgcn_cvt_off_f32_i4(wk >> 24), D2, V);
          V = fmaf(__builtin_amdgcn_cvt_off_f32_i4(wk >> 28), D3, V);
          acc += ldexpf(V, (int)((q.e >> (4 * k)) & 15u));
        }
      }
      // Sum the row over its 4 lanes; lane g == 0 stores the unit's partial.
      acc += dpp<0xB1>(acc);
      acc += dpp<0x4E>(acc);
      const int64_t row = (int64_t)kRowsPerSlab * sl + rho;
      const uint32_t poff = (g == 0 && row < Mp) ? (uint32_t)(u * Mp + row) * 4u : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), prsrc, poff, 0, 0);
    };

    // A wave's first two slabs are fixed (their loads went out before the
    // build); after that it takes the next slab of the segment from a counter
    // in LDS.  The SIMDs favour their older waves, so with a fixed share the
    // younger waves finished several microseconds later; taking slabs on demand
    // lets every wave finish within about one slab of the others.  Indices a
    // wave takes only grow, so once one is past the segment all later ones are.
    // Two register sets alternate, each load issued two slabs ahead of its use;
    // loads past the segment read harmless words (or zeros past the buffer).
    auto grab = [&]() -> int {
      int v = 0;
      if (lane == 0) v = atomicAdd(&sm.next_slab, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    int i0 = s_first, i1 = s_first + kWaves;
    while (i0 < sb) {
      const int i2 = grab(), i3 = grab();
      Slab Bq[2] = {load(i2), load(i3)};
      run(A[0], i0);
      const int i4 = grab();
      A[0] = load(i4);
      if (i1 < sb) run(A[1], i1);
      const int i5 = grab();
      A[1] = load(i5);
      if (i2 < sb) run(Bq[0], i2);
      if (i3 < sb) run(Bq[1], i3);
      i0 = i4;
      i1 = i5;
    }
    it = seg_end;
    mi = mn;
    u = un;
    sa = 0;
  }
}

static_assert(kSlots == panel_blocks(12), "a column unit is one packed panel");
int64_t units_of(const seedlm_matrix* h) { return h->np; }

bool fill_group12(const seedlm_matrix* const* hs, const void* const* xs, void* const* ys,
                  float* const* partials, int n, LutGroup& grp) {
  if (n < 1 || n > kMaxGroup) return false;
  grp = LutGroup{};
  grp.n = n;
  for (int i = 0; i < n; ++i) {
    const seedlm_matrix* h = hs[i];
    if (!h->is_3bit() || h->bytes >= 0x80000000ull) return false;
    if (h->Mp >= (1 << 27) || h->cols >= (1 << 30)) return false;
    const int64_t units = units_of(h);
    if (units * h->Mp * 4 >= (1LL << 31)) return false;  // partial offsets are 32-bit
    LutMatrix& M = grp.m[i];
    M.words = static_cast<const uint32_t*>(h->d_buf);
    M.x = xs[i];
    M.partial = partials[i];
    M.y = ys[i];
    M.words_bytes = (uint32_t)h->bytes;
    M.exp_off = (uint32_t)h->exp_off;
    M.Mp = (int)h->Mp;
    M.rows = (int)h->rows;
    M.cols = (int)h->cols;
    M.nb = (int)h->nb;
    M.np = (int)units;
    M.slabs = (int)((h->Mp + kRowsPerSlab - 1) / kRowsPerSlab);
  }
  // The partials hold 2^g sum_j (t_j/16) D_j with g = e + 15, and the window
  // values z - 2^15 are 2^15 times the entries of U: 2^-15 * 2^-15 * 16.
  grp.scale = 0x1p-26f;
  return split_group(grp, kBuildCost);
}

}  // namespace

// One fp32 partial per (column unit, padded row).
int64_t lut12_partial_floats(const seedlm_matrix* h) { return units_of(h) * h->Mp; }

int launch_gemv_lut12_group(const seedlm_matrix* const* hs, const void* const* xs,
                            void* const* ys, float* const* partials, int n, int xdt, int ydt,
                            hipStream_t s, int phases) {
  LutGroup grp;
  if (!fill_group12(hs, xs, ys, partials, n, grp)) return SEEDLM_E_UNSUPPORTED;
  if (phases & 1) {
    hipEvent_t e0, e1;
    main_launch_events(&e0, &e1);
    if (xdt == SEEDLM_F32)
      hipExtLaunchKernelGGL((gemv_lut12_kernel<float>), dim3((unsigned)grp.grid), dim3(kThreads),
                            0, s, e0, e1, 0, grp);
    else
      hipExtLaunchKernelGGL((gemv_lut12_kernel<__half>), dim3((unsigned)grp.grid), dim3(kThreads),
                            0, s, e0, e1, 0, grp);
    SEEDLM_HIP_CHECK(hipGetLastError());
  }
  if (phases & 2) return launch_reduce(grp, ydt, s);
  return SEEDLM_OK;
}

}  // namespace seedlm
