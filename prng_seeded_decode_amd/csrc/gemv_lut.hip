// Batch-1 fused decode-GEMV for the 4-bit format (C=8, P=3, K=16).
//
// SeedLM's inference step fetches each block's seed s and coefficients t, rebuilds
// the block's weights from the LFSR output and uses them at once (paperhub.cn
// rebuttal text before Eq. (1); blocks of C weights = 2^e U(s) t, atlas.scime.ai
// "Approach").  This kernel never forms the weights.  It uses the sliding-window
// structure of the 16-bit Fibonacci LFSR instead:
//
//   state z_n = sum_k b[n+k] 2^k for one bit stream b (b[0..15] = seed bits),
//   column j of U holds states z_{8j} .. z_{8j+7}, so for one block
//   D_j = sum_i x_i (z_{8j+i} - 2^15) = sum_{m<23} b[8j+m] c_m - 2^15 sum_i x_i,
//   c_m = sum_{i+k=m, i<8, k<16} x_i 2^k.
//   With stream bytes B_0..B_4 (B_0, B_1 = seed bytes):
//   D_j = L0[B_j] + 2 c_7 B_{j+1} + L2[B_{j+2}],
//   L0[v] = sum_{k<8} bit_k(v) c_k - 2^15 sum_i x_i,  L2[v] = sum_{k<7} bit_k(v) c_{16+k}
//   (bits 8..15 of the window have c_m = 2^(m-7) c_7, so the middle byte enters
//   linearly).  The block adds 2^(e-15) sum_j t_j D_j to its row.
//
// Per panel (32 blocks = 256 columns) the workgroup builds L0 and L2 for the
// panel's 32 column blocks in LDS, component-major so that lanes working on
// different slots read different banks.  Stream bytes B_2..B_4 come from GF(2)
// tables (ext(s) = T0[s & 255] ^ T1[s >> 8]; the LFSR is linear over GF(2)),
// replicated per slot for the same reason, or -- TABLE variant -- from a
// 2^16-entry table of extension bits in global memory (L2/MALL resident).
//
// LDS: region A row v = [L0'[v] for slots 0..31 | T1[v] x32], region B row v =
// [T0[v] x16 | TC[v] x16 | L2[v] for slots 0..31]; 256 B per row, so one
// v_perm_b32 turns a byte and a per-lane constant into a row/column address, and
// L0'[B1] + T1[B1] come back from a single ds_read2_b32.  The 16-copy tables
// cost a 2-way bank conflict, which LDS bandwidth has room for.
//
// Per block the arithmetic is arranged to keep VALU work low:
//   * TC[v] is the coefficient byte v = (t1 << 4 | t0) as the fp16 pair
//     (t0/16, t1/16), used directly by v_fma_mix_f32 and v_dot2_f32_f16, and
//     t2/16 is one v_cvt_off_f32_i4 of the word's top byte (the instruction
//     turns a signed nibble into nibble/16); every coefficient carries the
//     same 1/16, an exact power of two that the panel reduction's scale undoes;
//   * T1[v] carries v in its top byte, so ext = T0[B0] ^ T1[B1] holds
//     (B2, B3, B4, B1) and one v_perm_b32 makes the fp16 pair
//     (1024 + B1, 1024 + B2) (0x64 is the fp16 exponent of 1024); then
//     t0 (1024 + B1) + t1 (1024 + B2) is one exact v_dot2_f32_f16, and
//     t2 (1024 + B3) one v_fma_mix_f32;
//   * L0' = L0 - 2048 c_7 removes the 1024 offsets again:
//     sum_j t_j D_j = sum_j t_j (L0'[B_j] + L2[B_{j+2}])
//                     + 2 c_7 sum_j t_j (1024 + B_{j+1}).
//
// Lane mapping: lane = 8*rho + g; the lane owns row r0+rho and slot group g
// (slots 4g..4g+3) and reads the group's four words with one 16-byte load.  The
// packed layout rotates each group by the row index, so the four rows of a
// half-wave touch 32 different slots at every step.  Each block's work is
// issued in three stages (GF(2) reads, table reads, arithmetic) over the four
// words of a lane, so the LDS latency of one block hides behind the others.  A
// row's partial sum is reduced over its 8 lanes with DPP and written per panel;
// reduce_panels_kernel adds the panels in a fixed order (deterministic).
#include "lfsr_device.h"
#include "lut_common.h"

namespace seedlm {
namespace {

constexpr int kThreads = 1024;  // 16 waves: 4 per SIMD
constexpr int kWaves = kThreads / 64;
#ifndef SEEDLM_LUT_NS
#define SEEDLM_LUT_NS 1
#endif
constexpr int kNS = SEEDLM_LUT_NS;  // slabs per processing call (1 or 2)
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

struct Smem {
  uint32_t A[256][64];  // [L0' (32 slots) | T1 (32 copies)]
  uint32_t B[256][64];  // [T0 (16 copies) | TC (16 copies) | L2 (32 slots)]
  float xs[256];
  float c7x2[32];
  uint32_t gf2[512];    // T0 then T1, staged before replication
};
constexpr int kColT0 = 0, kColTC = 16, kColL2 = 32;  // column bases in region B
constexpr uint32_t kRegionB = 65536;  // byte offset of B inside Smem

// Cost model of the work split: a panel's table build costs about as much as
// kBuildCost slabs of 8 rows.
constexpr int64_t kBuildCost = 51;


__device__ void build_panel_lut(Smem& sm, float xval) {
  // xval: this thread's x value of the panel (threads 0..255), loaded ahead.
  const int tid = threadIdx.x;
  if (tid < 256) sm.xs[tid] = xval;
  __syncthreads();
  // Thread -> (slot, value group): kNV consecutive table rows per thread; the
  // low kLB bits of the row index come from small tables built by doubling,
  // the high bits are fixed per thread.  Half of the workgroup builds, 16 rows
  // per thread: the build's cost is its instructions per wave, and 8 waves of
  // 16 rows issue about half of what 16 waves of 8 rows do (1-2% of the launch).
  constexpr int kBuildThreads = 512;
  constexpr int kNV = 256 / (kBuildThreads / 32);
  constexpr int kLB = 4;
  static_assert((1 << kLB) == kNV && kBuildThreads <= kThreads, "16 rows per thread");
  if (tid >= kBuildThreads) return;
  const int slot = tid & 31, vg = tid >> 5;
  float xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = sm.xs[slot * 8 + i];
  // c_m = sum_{i+k=m, i<8, k<16} x_i 2^k: doubling for m <= 7 (only c_0..c_7
  // are needed there), halving downwards for m = 22..16.
  float c[23];
  c[0] = xv[0];
#pragma unroll
  for (int m = 1; m < 8; ++m) c[m] = fmaf(2.f, c[m - 1], xv[m]);
  c[22] = 32768.f * xv[7];
#pragma unroll
  for (int m = 21; m >= 16; --m) c[m] = fmaf(0.5f, c[m + 1], 32768.f * xv[m - 15]);
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) S += xv[i];
  float B0 = -32768.f * S - 2048.f * c[7], B2 = 0.f;
#pragma unroll
  for (int k = kLB; k < 8; ++k) {
    if ((vg >> (k - kLB)) & 1) {
      B0 += c[k];
      if (k < 7) B2 += c[16 + k];
    }
  }
  float A0[kNV], A2[kNV];
  A0[0] = A2[0] = 0.f;
#pragma unroll
  for (int n = 1; n < kNV; ++n) {
    const int low = __builtin_ctz(n), rest = n & (n - 1);
    A0[n] = A0[rest] + c[low];
    A2[n] = A2[rest] + c[16 + low];
  }
#pragma unroll
  for (int n = 0; n < kNV; ++n) {
    const int v = vg * kNV + n;
    sm.A[v][slot] = __float_as_uint(A0[n] + B0);
    sm.B[v][kColL2 + slot] = __float_as_uint(A2[n] + B2);
  }
  if (vg == 0) sm.c7x2[slot] = 2.f * c[7];
}

template <typename XT, bool kGlobalTable>
__global__ void __launch_bounds__(kThreads, 1)
    gemv_lut_kernel(const LutGroup grp, const uint32_t* __restrict__ ext_table) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rho = lane >> 3, g = lane & 7;
  const uint8_t* lds = reinterpret_cast<const uint8_t*>(&sm);

  // Each workgroup takes one contiguous range of the group's work items; the
  // host split them so that every range has about the same cost.
  const int64_t begin = grp.bounds[blockIdx.x];
  const int64_t end = grp.bounds[blockIdx.x + 1];
  // Where `begin` lies: matrix mi, panel pp, first slab sa.  This is the only
  // division of the loop; each later segment starts at the next panel.
  int mi = 0;
  while (mi + 1 < grp.n && begin >= grp.m[mi + 1].item_begin) ++mi;
  int pp = 0, sa = 0;
  if (begin < end) {
    const uint32_t local = (uint32_t)(begin - grp.m[mi].item_begin);
    const uint32_t slabs = (uint32_t)grp.m[mi].slabs;
    pp = (int)(local / slabs);
    sa = (int)(local - (uint32_t)pp * slabs);
  }
  // The x of a segment's panel is loaded one segment ahead (threads 0..255
  // hold one raw value each) with a buffer load whose out-of-range offset
  // reads zero, so no branch or select follows the load and nothing waits on
  // it until the table build that uses it.
  auto fetch_x = [&](int m2, int p2, bool valid) -> uint32_t {
    const LutMatrix& N = grp.m[m2];
    const int64_t c = (int64_t)p2 * 256 + tid;
    const uint32_t off = (valid && tid < 256 && c < N.cols) ? (uint32_t)c * sizeof(XT)
                                                           : 0x80000000u;
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
  uint32_t x_next = fetch_x(mi, pp, begin < end);

  // Copies of the GF(2) tables and of TC (built once per launch): values
  // staged, then replicated with 16-byte writes where consecutive lanes write
  // consecutive addresses (no bank conflicts).  T1's top byte is its index.
  if (tid < 512) {
    const uint32_t u = tid & 255;
    sm.gf2[tid] = tid < 256 ? ext_bits<uint32_t>(u) & 0x00FFFFFFu
                            : (ext_bits<uint32_t>(u << 8) & 0x00FFFFFFu) | (u << 24);
  }
  __syncthreads();
  // T1: 256 rows x 8 uint4 (32 copies); T0 and TC: 256 rows x 4 uint4 each.
#pragma unroll
  for (int k = 0; k < 4096 / kThreads; ++k) {
    const int e = tid + k * kThreads;  // k < 2: T1; k >= 2: T0 and TC
    uint32_t val;
    uint4* dst;
    if (e < 2048) {
      const int u = e >> 3, part = e & 7;
      val = sm.gf2[256 + u];
      dst = reinterpret_cast<uint4*>(&sm.A[u][32]) + part;
    } else {
      const int f = e - 2048, u = f >> 3, part = f & 7;
      if (part < 4) {
        val = sm.gf2[u];
        dst = reinterpret_cast<uint4*>(&sm.B[u][kColT0]) + part;
      } else {  // (t0, t1)/16 of the coefficient byte u, as an fp16 pair (exact)
        const int lo = u & 15, hi = u >> 4;
        const __half h0 = __float2half((float)(lo - ((lo & 8) << 1)) * 0.0625f);
        const __half h1 = __float2half((float)(hi - ((hi & 8) << 1)) * 0.0625f);
        val = (uint32_t)__half_as_ushort(h0) | ((uint32_t)__half_as_ushort(h1) << 16);
        dst = reinterpret_cast<uint4*>(&sm.B[u][kColTC]) + (part - 4);
      }
    }
    *dst = make_uint4(val, val, val, val);
  }

  // Slots of this lane's four words: slot_j = 4g + ((j + row) & 3); slabs start
  // at multiples of 8 rows, so row & 3 == rho & 3.
  uint32_t lcA[4], lcB[4], lcT0[4], lcTC[4];
  int slotj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    slotj[j] = 4 * g + ((j + rho) & 3);
    lcA[j] = (uint32_t)slotj[j] * 4u;
    lcB[j] = ((uint32_t)(kColL2 + slotj[j]) * 4u) | kRegionB;
    lcT0[j] = ((uint32_t)(kColT0 + (slotj[j] & 15)) * 4u) | kRegionB;
    lcTC[j] = ((uint32_t)(kColTC + (slotj[j] & 15)) * 4u) | kRegionB;
  }



  for (int64_t it = begin; it < end;) {
    const LutMatrix& M = grp.m[mi];
    const int64_t Mp = M.Mp, np = M.np;
    const int slabs = M.slabs;
    const int64_t p = pp;
    const int64_t pstart = M.item_begin + p * slabs;
    const int64_t seg_end = pstart + slabs < end ? pstart + slabs : end;
    const int sb = (int)(seg_end - pstart);
    int mn = mi, pn = pp + 1;  // the next segment's panel
    if (pn == M.np) {
      pn = 0;
      ++mn;
    }
    const int Wp = (int)panel_stored_width(p, M.nb, kPanelBlocks);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)M.words, 0, (int)M.words_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t prsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)M.partial, 0, (int)(np * Mp * 4), 0x00020000);
    const uint32_t lane_base =
        4 * g < Wp ? (uint32_t)(p * Mp * kPanelBlocks + rho * Wp + 4 * g) * 4u : 0x80000000u;
    const uint32_t slab_stride = 8u * (uint32_t)Wp * 4u;
    auto load = [&](int sl) {
      return __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_base + (uint32_t)sl * slab_stride,
                                                   0, 0);
    };
    // This wave's slabs are s_first, s_first + 16, ...; the first two loads
    // go out before the table build so that their latency overlaps it.
    const int s_first = sa + wave;
    v4u A[2] = {load(s_first), load(s_first + kWaves)};
    const uint32_t x_this = x_next;
    x_next = fetch_x(mn < grp.n ? mn : mi, pn, seg_end < end);
    __syncthreads();  // previous panel's tables no longer in use
    build_panel_lut(sm, x_value(x_this));
    __syncthreads();
    float c7j[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c7j[j] = sm.c7x2[slotj[j]];

    // Lanes outside the panel's width get an out-of-range base: their loads
    // return zero words (t = 0, no contribution).  Offsets grow by one slab
    // stride per step, so no per-load bounds logic is needed.
    const uint32_t pstore = g == 0 ? (uint32_t)(p * Mp + rho) * 4u : 0x80000000u;

    // kNS slabs per call (4*kNS blocks per lane): each stage issues the LDS
    // reads of all the call's blocks before the first use.  Each slab's row sum
    // is reduced over its 8 lanes and stored as the panel partial of that row.
    auto run = [&](const v4u (&q)[kNS], int sl0, int nvalid) {
      constexpr int NB = 4 * kNS;
      uint32_t w[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) w[k] = q[k >> 2][k & 3];
      // Stage 1: GF(2) halves, coefficient pairs and the seed-byte L0' values.
      float l0b0[NB], l0b1[NB];
      uint32_t ext[NB], tcv[NB];
      if (kGlobalTable) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          l0b0[k] = lds_at<float>(lds, lut_addr<0>(w[k], lcA[k & 3]));
          l0b1[k] = lds_at<float>(lds, lut_addr<1>(w[k], lcA[k & 3]));
          tcv[k] = lds_at<uint32_t>(lds, lut_addr<2>(w[k], lcTC[k & 3]));
          ext[k] = ext_table[w[k] & 0xFFFFu];
        }
      } else {
        uint32_t t0v[NB], t1v[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          const uint32_t a1 = lut_addr<1>(w[k], lcA[k & 3]);
          l0b0[k] = lds_at<float>(lds, lut_addr<0>(w[k], lcA[k & 3]));
          t0v[k] = lds_at<uint32_t>(lds, lut_addr<0>(w[k], lcT0[k & 3]));
          l0b1[k] = lds_at<float>(lds, a1);
          t1v[k] = lds_at<uint32_t>(lds, a1 + 128);
          tcv[k] = lds_at<uint32_t>(lds, lut_addr<2>(w[k], lcTC[k & 3]));
        }
        __builtin_amdgcn_sched_barrier(0);  // all stage-1 reads issue before any use
#pragma unroll
        for (int k = 0; k < NB; ++k) ext[k] = t0v[k] ^ t1v[k];
      }
      // Stage 2: table values of the extension bytes B_2..B_4.
      float l0b2[NB], l2b2[NB], l2b3[NB], l2b4[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        l0b2[k] = lds_at<float>(lds, lut_addr<0>(ext[k], lcA[k & 3]));
        l2b2[k] = lds_at<float>(lds, lut_addr<0>(ext[k], lcB[k & 3]));
        l2b3[k] = lds_at<float>(lds, lut_addr<1>(ext[k], lcB[k & 3]));
        l2b4[k] = lds_at<float>(lds, lut_addr<2>(ext[k], lcB[k & 3]));
      }
      __builtin_amdgcn_sched_barrier(0);
      // Stage 3: arithmetic.
      float acc[kNS];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int j = k & 3;
        const uint32_t wk = w[k];
        const half2v tc = __builtin_bit_cast(half2v, tcv[k]);  // (t0, t1)/16
        // (1024 + B1, 1024 + B2) and (1024 + B3, 0) as fp16 pairs
        const half2v p12 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(ext[k], 0x64646464u, 0x01040007u));
        const half2v p3 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(ext[k], 0x64646464u, 0x0C0C0005u));
        const float t2 = __builtin_amdgcn_cvt_off_f32_i4(wk >> 24);  // t2/16
        const float mid = __builtin_amdgcn_fdot2(tc, p12, __builtin_fmaf(t2, (float)p3[0], 0.f), false);
        float V = t2 * (l0b2[k] + l2b4[k]);
        V = fmaf((float)tc[0], l0b0[k] + l2b2[k], V);
        V = fmaf((float)tc[1], l0b1[k] + l2b3[k], V);
        V = fmaf(c7j[j], mid, V);
        const float part = ldexpf(V, (int)(wk >> 28));
        acc[k >> 2] = j == 0 ? part : acc[k >> 2] + part;
      }
      // Sum each row over its 8 lanes (xor 1, xor 2, then mirror within 8).
#pragma unroll
      for (int h = 0; h < kNS; ++h) {
        acc[h] += dpp<0xB1>(acc[h]);
        acc[h] += dpp<0x4E>(acc[h]);
        acc[h] += dpp<0x141>(acc[h]);
        if (h < nvalid)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[h]), prsrc,
                                                pstore + (uint32_t)(sl0 + h * kWaves) * 32u, 0, 0);
      }
    };

    // Two register sets alternate (A: slabs 0, 1 of each group of four, B:
    // slabs 2, 3), each load issued two slabs ahead of its use; nothing is
    // copied at the back edge, so a wait never covers a load younger than the
    // one it needs.  Loads past the panel read harmless words (or zeros past
    // the buffer) and are not used.
    auto group = [&](int s0) {
      v4u Bq[2] = {load(s0 + 2 * kWaves), load(s0 + 3 * kWaves)};
      const int n0 = min(4, (sb - s0 + kWaves - 1) / kWaves);  // valid slabs of the group
      if constexpr (kNS == 2) {
        run(A, s0, min(n0, 2));
        A[0] = load(s0 + 4 * kWaves);
        A[1] = load(s0 + 5 * kWaves);
        if (n0 > 2) run(Bq, s0 + 2 * kWaves, n0 - 2);
      } else {
        run({A[0]}, s0, 1);
        A[0] = load(s0 + 4 * kWaves);
        if (n0 > 1) run({A[1]}, s0 + kWaves, 1);
        A[1] = load(s0 + 5 * kWaves);
        if (n0 > 2) run({Bq[0]}, s0 + 2 * kWaves, 1);
        if (n0 > 3) run({Bq[1]}, s0 + 3 * kWaves, 1);
      }
    };
    // The wave's full groups run in a loop whose body holds no test on the
    // slab count, so it compiles to one straight block that the scheduler can
    // interleave freely (2-3% faster than testing every slab); the last group,
    // which may hold fewer than four of the wave's slabs, runs after it.
    int s0 = s_first;
    for (; s0 + 4 * kWaves < sb; s0 += 4 * kWaves) group(s0);
    if (s0 < sb) group(s0);
    it = seg_end;
    mi = mn;
    pp = pn;
    sa = 0;
  }
}

bool fill_group(const seedlm_matrix* const* hs, const void* const* xs, void* const* ys,
                float* const* partials, int n, LutGroup& grp) {
  if (n < 1 || n > kMaxGroup) return false;
  grp = LutGroup{};
  grp.n = n;
  for (int i = 0; i < n; ++i) {
    const seedlm_matrix* h = hs[i];
    if (!h->is_4bit() || h->bytes >= 0x80000000ull) return false;
    if (h->Mp >= (1 << 28) || h->cols >= (1 << 30)) return false;
    if (h->np * h->Mp * 4 >= (1LL << 31)) return false;  // partial offsets are 32-bit
    LutMatrix& M = grp.m[i];
    M.words = static_cast<const uint32_t*>(h->d_buf);
    M.x = xs[i];
    M.partial = partials[i];
    M.y = ys[i];
    M.words_bytes = (uint32_t)h->bytes;
    M.Mp = (int)h->Mp;
    M.rows = (int)h->rows;
    M.cols = (int)h->cols;
    M.nb = (int)h->nb;
    M.np = (int)h->np;
    M.slabs = (int)(h->Mp / 8);
  }
  // The partials hold 2^g sum_j (t_j/16) D_j with g = e + 15, and the window
  // values z - 2^15 are 2^15 times the entries of U: 2^-15 * 2^-15 * 16.
  grp.scale = 0x1p-26f;
  return split_group(grp, kBuildCost);
}

template <typename XT, bool kGT>
void launch_main(const LutGroup& grp, const uint32_t* table, hipStream_t s) {
  hipEvent_t e0, e1;
  main_launch_events(&e0, &e1);
  hipExtLaunchKernelGGL((gemv_lut_kernel<XT, kGT>), dim3((unsigned)grp.grid), dim3(kThreads), 0,
                        s, e0, e1, 0, grp, table);
}

}  // namespace

// One fp32 partial per (panel, padded row).
int64_t lut_partial_floats(const seedlm_matrix* h) { return h->np * h->Mp; }

int launch_gemv_lut_group(const seedlm_matrix* const* hs, const void* const* xs, void* const* ys,
                          float* const* partials, int n, int xdt, int ydt,
                          const uint32_t* ext_table, hipStream_t s, int phases) {
  LutGroup grp;
  if (!fill_group(hs, xs, ys, partials, n, grp)) return SEEDLM_E_UNSUPPORTED;
  if (phases & 1) {
    const bool global_table = ext_table != nullptr;
    if (xdt == SEEDLM_F32) {
      if (global_table) launch_main<float, true>(grp, ext_table, s);
      else launch_main<float, false>(grp, ext_table, s);
    } else {
      if (global_table) launch_main<__half, true>(grp, ext_table, s);
      else launch_main<__half, false>(grp, ext_table, s);
    }
    SEEDLM_HIP_CHECK(hipGetLastError());
  }
  if (phases & 2) return launch_reduce(grp, ydt, s);
  return SEEDLM_OK;
}

}  // namespace seedlm
