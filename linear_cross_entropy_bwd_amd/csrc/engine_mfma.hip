// bf16 matrix-core engine for gfx950: the three contractions of the fused
// linear cross-entropy on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
//   logits  Z^T[j, t] = sum_k W[j, k] H[t, k]    A = W   (k-major), B = H   (k-major)
//   dH      dH[t, k]  = sum_j G[t, j] W[j, k]    A = G   (k-major), B = W   (n-major)
//   dW      dW[j, k]  = sum_t G[t, j] H[t, k]    A = G^T (m-major), B = H   (n-major)
//
// In the one-pass backward G = diag(F) P' (one factor per token row): dH takes
// P' as A and scales its output rows by F, dW takes P'^T as A and diag(F) H,
// a bf16 copy written beforehand, as B.
//
// One 256x256 output tile per 256-thread block (4 waves, 2x2, 128x128 per
// wave = 4x4 MFMA tiles of 32x32).  K advances 64 at a time.  Operand tiles
// go from global memory straight into LDS with 16-byte loads (no register
// staging; buffer loads inside the operands, direct global->LDS loads at
// their edges) through a ring of five 32 KB operand-stage slots, so the
// A operand is fetched two stages and the B operand one stage ahead of the
// MFMAs (see tile_loop).  Tiles whose k index is contiguous in memory sit in
// LDS as [256 rows][64 k] and feed the fragments with 16-byte reads; tiles
// whose k index is strided (the n-major W of dH, the m-major G^T and n-major H
// of dW) sit in LDS as they are in memory, [64 k][256 mn], and are transposed
// on the way into the fragments by the gfx950 LDS transpose read
// (ds_read_b64_tr_b16).  Both layouts XOR-swizzle their 16-byte chunks so
// that the fragment reads hit distinct LDS banks.  Loads that fall outside an
// operand read a 16-byte block of zeros instead.
//
// The logits are computed transposed (vocabulary on the MFMA rows, tokens on
// the lanes) so that each lane holds 64 vocabulary entries of the same token:
// the per-token max and sum-exp over a 128-wide vocabulary group need one
// cross-lane step.  The epilogue stores exp(z - group max), or in the
// one-pass backward exp(z - r) against a per-row reference r, in bf16 into the
// chunk's buffer; the full logits never leave registers.
//
// Consecutive workgroups are dispatched round-robin over the 8 XCDs; block
// ids are remapped so that each XCD walks a contiguous range of tiles, and
// tiles are ordered so that neighbours share an operand tile in that XCD's L2.
#include "device_util.h"
#include "flce_internal.h"

namespace flce {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int TM = 256;       // tile rows (MFMA M)
constexpr int TN = 256;       // tile cols (MFMA N)
constexpr int TK = 64;        // k per LDS stage: 128-byte row segments, whole cache lines
constexpr int kSlots = 5;     // LDS ring of operand-stage slots: 5 x 32 KB
constexpr int kThreads = 256;
constexpr int kStageElems = TM * TK;  // one operand, one stage: 32 KB

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef int v8i32 __attribute__((ext_vector_type(8)));
#define FLCE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Source of every out-of-range 16-byte load.
__device__ __attribute__((aligned(16))) unsigned int g_zero16[4] = {0u, 0u, 0u, 0u};

struct Operand {
  const bf16_t* ptr;
  int64_t ld;        // elements between consecutive rows in memory
  int64_t mn_bound;  // rows (k-major) / columns (mn-major) that exist
  int64_t k_bound;   // k values that exist (absolute index)
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Stage layouts in LDS (bf16 elements, one operand, one stage = 256 x 64):
//  k-major : row R (= mn) of 64 k = 8 chunks of 8 k; position p of row R
//            holds k-chunk p ^ ((R >> 1) & 7).
//  mn-major: row k of 256 mn = 32 chunks of 8 mn; position p of row k holds
//            mn-chunk p ^ (4 (k & 3)).
// A stage is filled by 8 direct 16-byte loads per wave: load i of wave w
// fills LDS bytes [1024 (8w + i), +1024), lane L landing at +16 L, i.e.
//  k-major : rows R = 64 w + 8 i + L / 8, position L % 8;
//  mn-major: rows k = 16 w + 2 i + L / 32, position L % 32.
// The swizzle depends on i only through its parity, so a lane needs two byte
// offsets (even / odd i) relative to a per-load uniform base.
constexpr int kLoadsPerStage = 8;  // per wave and operand

template <bool KMAJ>
__device__ __forceinline__ void lane_load_offsets(int64_t ld, uint32_t (&off)[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    if (KMAJ) {
      const int kc = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7);
      off[par] = static_cast<uint32_t>((lane >> 3) * ld * 2 + 16 * kc);
    } else {
      const int c = (lane & 31) ^ (4 * ((2 * par + (lane >> 5)) & 3));
      off[par] = static_cast<uint32_t>((lane >> 5) * ld * 2 + 16 * c);
    }
  }
}

// Loads I0 .. I0 + CNT - 1 of a wave's share of one operand-stage.
// Interior stage: every load in bounds, issued as buffer loads: one
// descriptor per call whose base is the wave's first row of the stage, the
// row step of load i as the scalar offset and the lane's part as a 32-bit
// vector offset (lane and row offsets stay below 2^31 for leading dimensions
// below 2^24, which the plan enforces), so only 4 bytes of each lane's
// address live in vector registers.
template <int I0, int CNT, bool KMAJ>
__device__ __forceinline__ void load_stage_fast(const Operand& op, int64_t mn0, int64_t k0, bf16_t* lds,
                                                const uint32_t (&off)[2]) {
  const int w = wave_id();
  // the row offset is uniform; saying so keeps the descriptor in scalar
  // registers (the compiler otherwise wraps each load in a waterfall loop)
  const int64_t first0 = KMAJ ? (mn0 + 64 * w) * op.ld + k0 : (k0 + 16 * w) * op.ld + mn0;
  const uint64_t fu = static_cast<uint64_t>(first0);
  const int64_t first = static_cast<int64_t>(
      (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(fu >> 32))) << 32) |
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(fu))));
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(op.ptr + first), 0, 0x7fffffff, 0x00020000);
  const uint32_t row_bytes = static_cast<uint32_t>(op.ld) * 2u;
#pragma unroll
  for (int i = I0; i < I0 + CNT; ++i) {
    const uint32_t soff = static_cast<uint32_t>(KMAJ ? 8 * i : 2 * i) * row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FLCE_LDS(lds + (w * kLoadsPerStage + i) * 512), 16, off[i & 1], soff,
                                             0, 0);
  }
}

// Edge stage: per-lane bounds; out-of-range lanes read 16 zero bytes.
template <int I0, int CNT, bool KMAJ>
__device__ __forceinline__ void load_stage_edge(const Operand& op, int64_t mn0, int64_t k0, bf16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const unsigned int* zero = g_zero16;
#pragma unroll
  for (int i = I0; i < I0 + CNT; ++i) {
    const int b = w * kLoadsPerStage + i;
    const void* src;
    if (KMAJ) {
      const int R = b * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ ((R >> 1) & 7);
      const int64_t mn = mn0 + R, k = k0 + kc * 8;
      const bool ok = mn < op.mn_bound && k + 8 <= op.k_bound;
      src = ok ? static_cast<const void*>(op.ptr + mn * op.ld + k) : static_cast<const void*>(zero);
    } else {
      const int kr = b * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (kr & 3));
      const int64_t k = k0 + kr, mn = mn0 + c * 8;
      const bool ok = k < op.k_bound && mn + 8 <= op.mn_bound;
      src = ok ? static_cast<const void*>(op.ptr + k * op.ld + mn) : static_cast<const void*>(zero);
    }
    __builtin_amdgcn_global_load_lds(src, FLCE_LDS(lds + b * 512), 16, 0, 0);
  }
}

template <int I0, int CNT, bool KMAJ>
__device__ __forceinline__ void load_stage(const Operand& op, int64_t mn0, int64_t k0, bf16_t* lds,
                                           const uint32_t (&off)[2]) {
  const bool interior = mn0 + TM <= op.mn_bound && k0 + TK <= op.k_bound;
  if (interior)
    load_stage_fast<I0, CNT, KMAJ>(op, mn0, k0, lds, off);
  else
    load_stage_edge<I0, CNT, KMAJ>(op, mn0, k0, lds);
}

// Per-lane LDS byte offsets of the fragment reads of a wave whose operand rows
// start at wbase (multiple of 128).  Fragment (subtile i, k-step ks) holds
// operand rows wbase + 32 i + (lane % 32) and k = 16 ks + 8 (lane / 32) + 0..7.
//  k-major : offset = fo[ks] + 4096 i            (one 16-byte read)
//  mn-major: offset = fo[i] + 8192 ks (+ 2048)   (two transpose reads: k + 0..3, k + 4..7)
template <bool KMAJ>
__device__ __forceinline__ void lane_frag_offsets(int wbase, uint32_t (&fo)[4]) {
  const int lane = threadIdx.x & 63;
  if (KMAJ) {
    const int r = lane & 31, h = lane >> 5;
    const int sw = (r >> 1) & 7;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) fo[ks] = static_cast<uint32_t>((wbase + r) * 128 + 16 * ((2 * ks + h) ^ sw));
  } else {
    // 16-lane groups: lane s of group g points at k = kb + s / 4, mn = nb + 4 (s % 4);
    // the transpose read hands lane s the 4 consecutive k of column nb + s.
    const int g = lane >> 4, s = lane & 15, q = s >> 2;
    const int low = 2 * (g & 1) + ((s & 3) >> 1);
    const int base = (8 * (g >> 1) + q) * 512 + 2 * wbase + 16 * low + 8 * (s & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) fo[i] = static_cast<uint32_t>(base + 64 * (i ^ q));
  }
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(FLCE_LDS(p)));
}

// Fragment (subtile i, k-step KS) of the operand whose stage starts at LDS
// byte address `slot`.  The k-major read is an ordinary LDS load.  The
// transpose reads are issued as inline assembly: the compiler does not
// separate the builtin's LDS access from the direct loads still filling other
// slots and would wait for every one of them (vmcnt(0)) before each read,
// which serializes loads and MFMAs.  The ordering these reads need is
// explicit instead: the stage barrier (all volatile asm keeps its order)
// before them, and wait_frags() between them and the MFMAs that use them.
template <bool KMAJ, int KS>
__device__ __forceinline__ bf16x8 read_frag(const bf16_t* lds, uint32_t slot, const uint32_t (&fo)[4], int i) {
  if constexpr (KMAJ) {
    const char* b = reinterpret_cast<const char*>(lds);
    return *reinterpret_cast<const bf16x8*>(b + fo[KS] + 4096 * i);
  } else {
    v4i16 lo, hi;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:%4"
        : "=&v"(lo), "=&v"(hi)
        : "v"(slot + fo[i]), "i"(8192 * KS), "i"(8192 * KS + 2048));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// XCD-aware remap: hardware block b runs on XCD b % 8; give XCD x the
// contiguous tile range [start(x), start(x) + count(x)).
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb) {
  const int64_t per = nb / 8, rem = nb % 8;
  const int64_t x = b % 8, i = b / 8;
  return x * per + (x < rem ? x : rem) + i;
}

// Tile coordinates of linear tile t in a tiles_m x tiles_n grid, walked in
// groups of group_m tile rows: inside a group the row index runs fastest, so
// a run of consecutive tiles covers a group_m x k block of the output and its
// operand tiles (group_m A tiles, k B tiles) are shared in L2.
__device__ __forceinline__ void tile_coords(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t group_m,
                                            int64_t& tm, int64_t& tn) {
  const int64_t per_group = group_m * tiles_n;
  const int64_t grp = t / per_group, in = t % per_group;
  const int64_t first = grp * group_m;
  const int64_t gm = tiles_m - first < group_m ? tiles_m - first : group_m;
  tm = first + in % gm;
  tn = in / gm;
}

struct Acc {
  floatx16 c[4][4];
};

struct Frags {
  bf16x8 a[4], b[4];
};

// Wait for every LDS read in flight and make the registers of the fragments
// read by inline assembly (the transposed operands) depend on that wait, so
// that no MFMA reading them is scheduled before it.  Fragments read by plain
// loads are tracked by the compiler, which waits for exactly what it needs.
template <bool A_KMAJ, bool B_KMAJ>
__device__ __forceinline__ void wait_frags(Frags& f) {
  if constexpr (!A_KMAJ && !B_KMAJ) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]),
                   "+v"(f.b[3]));
  } else if constexpr (!A_KMAJ) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]));
  } else if constexpr (!B_KMAJ) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
  }
}

// Wait until at most `n` operand-stages (8 direct loads each, per wave) are
// still in flight: s_waitcnt vmcnt(8 n), lgkmcnt and expcnt left alone (gfx9
// encoding: vmcnt bits [3:0] and [15:14]).
__device__ __forceinline__ void wait_stages(int n) {
  static_assert(kLoadsPerStage == 8, "vmcnt immediates assume 8 loads per operand-stage");
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x4F70); break;
    default: __builtin_amdgcn_s_waitcnt(0x4F78); break;
  }
}

// s_waitcnt vmcnt(N) for a compile-time N < 64, lgkmcnt and expcnt left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads(): the direct
// loads are waited for explicitly.  The wave's own LDS reads complete first,
// so that a slot the barrier frees is no longer being read by anyone.  The
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The workgroup's LDS: the ring of operand-stage slots of the main loop.
// After tile_loop returns, wave w may reuse bytes [8192 w, 8192 w + 8192) of
// every slot as private scratch: only its own direct loads ever wrote there
// (all drained), and no wave reads the ring after the last stage barrier.
__device__ __forceinline__ bf16_t (*ring())[kStageElems] {
  __shared__ __attribute__((aligned(16))) bf16_t lds[kSlots][kStageElems];
  return lds;
}
constexpr int kWaveScratchBytes = 8192;

// Placement inside one k-step of 16 MFMAs: fragment read f (A 0..3, then B
// 0..3) of the next k-step and direct load q issue after MFMA kReadAfter[f] and
// kLoadAfter[q] of the current one.
constexpr int kReadAfter[8] = {0, 1, 2, 3, 4, 5, 6, 7};
constexpr int kLoadAfter[4] = {8, 9, 10, 11};

// Main loop: acc += A[m0 .. m0+255, k_lo .. k_hi) * B[n0 .. n0+255, k_lo .. k_hi)^T
//
// LDS is a ring of 5 operand-stage slots of 32 KB (the whole 160 KB):
// operand-stage q (A_s is q = 2s, B_s is q = 2s + 1) lives in slot q % 5.
// Iteration j runs from one workgroup barrier to the next and computes stage
// j in four k-steps; the fragments of each k-step are read from LDS while the
// MFMAs of the previous one run.  At its start every wave has finished
// reading stage j-1, so the two slots that stage used are free: the
// iteration fills them with B_{j+1} and A_{j+2}, four direct loads per wave
// beside each k-step's MFMAs rather than in one burst:
//   k-step 0: MFMAs of k-step 3 of stage j-1 | reads of k-step 0 | B_{j+1} loads 0..3
//   k-step 1: MFMAs of k-step 0              | reads of k-step 1 | B_{j+1} loads 4..7
//   k-step 2: MFMAs of k-step 1              | reads of k-step 2 | A_{j+2} loads 0..3
//   k-step 3: MFMAs of k-step 2              | reads of k-step 3 | A_{j+2} loads 4..7
//   wait until only A_{j+2} may be in flight; barrier (stage j+1 has landed
//     for every wave, and every wave has read all of stage j)
// So A is fetched two stages and B one stage ahead of its use.  Stages past
// the end load zeros and are never consumed, so every iteration issues the
// same loads and the waits are constants.
//
// FP8 (both operands k-major, e4m3 bytes viewed as 16-bit pairs, so that
// loads, slots and offsets are those of bf16): a stage holds 128 fp8 values
// of k and runs as two 64-deep k-steps of v_mfma_f32_32x32x64_f8f6f4.  A
// lane's fp8 operand for k-step q is its bf16-layout fragments of k-steps 2q
// and 2q+1 side by side; the k order inside an MFMA does not matter as long
// as both operands share it, and each lane half still covers disjoint k.
//   k-step 0: MFMAs of k-step 1 of stage j-1 | reads of 0, 1 | B_{j+1} loads
//   k-step 1: MFMAs of k-step 0              | reads of 2, 3 | A_{j+2} loads
template <bool A_KMAJ, bool B_KMAJ, bool FP8 = false>
__device__ __forceinline__ void tile_loop(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int64_t k_lo,
                                          int64_t k_hi, Acc& acc) {
  static_assert(!FP8 || (A_KMAJ && B_KMAJ), "the fp8 loop takes k-major operands");
  bf16_t (*lds)[kStageElems] = ring();
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.0f;

  uint32_t offa[2], offb[2], foa[4], fob[4];
  lane_load_offsets<A_KMAJ>(A.ld, offa);
  lane_load_offsets<B_KMAJ>(B.ld, offb);
  lane_frag_offsets<A_KMAJ>(wm * 128, foa);
  lane_frag_offsets<B_KMAJ>(wn * 128, fob);

  const int64_t nk = (k_hi - k_lo + TK - 1) / TK;
  auto k_of = [&](int64_t st) { return st < nk ? k_lo + st * TK : k_hi; };  // past the end: zeros
  const uint32_t lds0 = lds_addr(lds[0]);

  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc.c[i][j], 0, 0, 0);
  };
  auto mma8_one = [&](int i, int j, const Frags& lo, const Frags& hi) {
    const v4i32 al = __builtin_bit_cast(v4i32, lo.a[i]), ah = __builtin_bit_cast(v4i32, hi.a[i]);
    const v4i32 bl = __builtin_bit_cast(v4i32, lo.b[j]), bh = __builtin_bit_cast(v4i32, hi.b[j]);
    const v8i32 a8 = __builtin_shufflevector(al, ah, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i32 b8 = __builtin_shufflevector(bl, bh, 0, 1, 2, 3, 4, 5, 6, 7);
    // formats 0, 0: both operands e4m3; no block scales
    acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc.c[i][j], 0, 0, 0, 0, 0, 0);
  };
  auto mma8 = [&](const Frags& lo, const Frags& hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma8_one(i, j, lo, hi);
  };
  auto next = [](int s, int d) { return s + d >= kSlots ? s + d - kSlots : s + d; };
  // One k-step: the 16 MFMAs on `cur` (when MMA), with the 8 fragment reads of
  // k-step KS into `nxt` and the direct loads load(0..3) placed between them
  // as kReadAfter / kLoadAfter say.  Scheduling barriers pin this order:
  // the scheduler sees no LDS read in the transpose reads' inline assembly
  // and would otherwise bunch them behind the MFMAs, leaving the next
  // k-step's wait uncovered.
  auto phase = [&](auto mma_on, const Frags& cur, Frags& nxt, int sa_, int sb_, auto ks, auto&& load) {
    constexpr bool MMA = decltype(mma_on)::value;
    constexpr int KS = decltype(ks)::value;
    const uint32_t slot_a = lds0 + sa_ * kStageElems * 2, slot_b = lds0 + sb_ * kStageElems * 2;
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (MMA)
        acc.c[m / 4][m % 4] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[m / 4], cur.b[m % 4], acc.c[m / 4][m % 4], 0, 0, 0);
      static_for<8>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        if constexpr (kReadAfter[f] == m) {
          if constexpr (f < 4)
            nxt.a[f] = read_frag<A_KMAJ, KS>(lds[sa_], slot_a, foa, f);
          else
            nxt.b[f - 4] = read_frag<B_KMAJ, KS>(lds[sb_], slot_b, fob, f - 4);
        }
      });
      static_for<4>([&](auto qc) {
        if constexpr (kLoadAfter[decltype(qc)::value] == m) load(qc);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Prologue: A_0, B_0, A_1 in flight; wait for A_0 and B_0.
  load_stage<0, kLoadsPerStage, A_KMAJ>(A, m0, k_of(0), lds[0], offa);
  load_stage<0, kLoadsPerStage, B_KMAJ>(B, n0, k_of(0), lds[1], offb);
  load_stage<0, kLoadsPerStage, A_KMAJ>(A, m0, k_of(1), lds[2], offa);
  wait_stages(1);
  stage_barrier();

  Frags f0, f1;
  int sa = 0, sb = 1;  // slots of stage j
  // One iteration.  FIRST: there is no k-step 3 of a previous stage to
  // finish.  FAST: both loaded stages lie inside their operands, so the loads
  // need no bounds checks and the iteration is one basic block.
  auto body = [&](int64_t j, auto first, auto fast) {
    constexpr bool kFirst = decltype(first)::value;
    constexpr bool kFast = decltype(fast)::value;
    bf16_t* slot_b = lds[next(sb, 2)];  // B_{j+1}: slot of A_{j-1}
    bf16_t* slot_a = lds[next(sa, 4)];  // A_{j+2}: slot of B_{j-1}
    const int64_t kb = k_of(j + 1), ka = k_of(j + 2);
    // direct load I0 + q of B_{j+1} / A_{j+2}, one per call
    auto load_b_at = [&](auto i0) {
      return [&](auto q) {
        constexpr int I = decltype(i0)::value + decltype(q)::value;
        if constexpr (kFast)
          load_stage_fast<I, 1, B_KMAJ>(B, n0, kb, slot_b, offb);
        else
          load_stage<I, 1, B_KMAJ>(B, n0, kb, slot_b, offb);
      };
    };
    auto load_a_at = [&](auto i0) {
      return [&](auto q) {
        constexpr int I = decltype(i0)::value + decltype(q)::value;
        if constexpr (kFast)
          load_stage_fast<I, 1, A_KMAJ>(A, m0, ka, slot_a, offa);
        else
          load_stage<I, 1, A_KMAJ>(A, m0, ka, slot_a, offa);
      };
    };
    auto load_b0 = load_b_at(std::integral_constant<int, 0>{});
    auto load_b4 = load_b_at(std::integral_constant<int, 4>{});
    auto load_a0 = load_a_at(std::integral_constant<int, 0>{});
    auto load_a4 = load_a_at(std::integral_constant<int, 4>{});
    if constexpr (!kFirst) wait_frags<A_KMAJ, B_KMAJ>(f1);
    phase(std::bool_constant<!kFirst>{}, f1, f0, sa, sb, std::integral_constant<int, 0>{}, load_b0);
    wait_frags<A_KMAJ, B_KMAJ>(f0);
    phase(std::true_type{}, f0, f1, sa, sb, std::integral_constant<int, 1>{}, load_b4);
    wait_frags<A_KMAJ, B_KMAJ>(f1);
    phase(std::true_type{}, f1, f0, sa, sb, std::integral_constant<int, 2>{}, load_a0);
    wait_frags<A_KMAJ, B_KMAJ>(f0);
    phase(std::true_type{}, f0, f1, sa, sb, std::integral_constant<int, 3>{}, load_a4);
    wait_stages(1);
    stage_barrier();
    sa = next(sa, 2);
    sb = next(sb, 2);
  };
  // Leading stages that lie wholly inside each operand; iteration j loads
  // B_{j+1} and A_{j+2}, so it is fast while j + 1 < inside_b and j + 2 < inside_a.
  auto inside = [&](const Operand& op, int64_t mn0) -> int64_t {
    if (mn0 + TM > op.mn_bound) return 0;
    const int64_t full = (op.k_bound - k_lo) / TK;
    return full < nk ? full : nk;
  };
  const int64_t ia = inside(A, m0), ib = inside(B, n0);
  const int64_t fast_end = ib - 1 < ia - 2 ? ib - 1 : ia - 2;
  if constexpr (!FP8) {
    if (nk > 0) body(0, std::true_type{}, std::false_type{});
    int64_t j = 1;
    for (; j < fast_end; ++j) body(j, std::false_type{}, std::true_type{});
    for (; j < nk; ++j) body(j, std::false_type{}, std::false_type{});
    if (nk > 0) {  // k-step 3 of the last stage
      wait_frags<A_KMAJ, B_KMAJ>(f1);
      mma(f1);
    }
  } else {
    Frags g0h, g1h;  // second halves of the two fp8 k-steps' operands (f0, f1 hold the first)
    // One fp8 k-step: its 16 MFMAs on (clo, chi) when MMA, the 16 fragment reads
    // of the next one (bf16-layout k-steps KS and KS + 1 into nlo, nhi), two after
    // each of the first 8 MFMAs, and the stage's 8 direct loads load(0..7), one
    // after each of the last 8, in the order scheduling barriers pin (as phase).
    auto phase8 = [&](auto mma_on, const Frags& clo, const Frags& chi, Frags& nlo, Frags& nhi, auto ks,
                      auto&& load) {
      constexpr bool MMA = decltype(mma_on)::value;
      constexpr int KS = decltype(ks)::value;
      const uint32_t slot_a = lds0 + sa * kStageElems * 2, slot_b = lds0 + sb * kStageElems * 2;
      static_for<16>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (MMA) mma8_one(m / 4, m % 4, clo, chi);
        if constexpr (m < 4) {
          nlo.a[m] = read_frag<A_KMAJ, KS>(lds[sa], slot_a, foa, m);
          nhi.a[m] = read_frag<A_KMAJ, KS + 1>(lds[sa], slot_a, foa, m);
        } else if constexpr (m < 8) {
          nlo.b[m - 4] = read_frag<B_KMAJ, KS>(lds[sb], slot_b, fob, m - 4);
          nhi.b[m - 4] = read_frag<B_KMAJ, KS + 1>(lds[sb], slot_b, fob, m - 4);
        } else {
          load(std::integral_constant<int, m - 8>{});
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto body8 = [&](int64_t j, auto first, auto fast) {
      constexpr bool kFirst = decltype(first)::value;
      constexpr bool kFast = decltype(fast)::value;
      bf16_t* slot_b = lds[next(sb, 2)];
      bf16_t* slot_a = lds[next(sa, 4)];
      const int64_t kb = k_of(j + 1), ka = k_of(j + 2);
      auto load_b = [&](auto q) {
        if constexpr (kFast)
          load_stage_fast<decltype(q)::value, 1, B_KMAJ>(B, n0, kb, slot_b, offb);
        else
          load_stage<decltype(q)::value, 1, B_KMAJ>(B, n0, kb, slot_b, offb);
      };
      auto load_a = [&](auto q) {
        if constexpr (kFast)
          load_stage_fast<decltype(q)::value, 1, A_KMAJ>(A, m0, ka, slot_a, offa);
        else
          load_stage<decltype(q)::value, 1, A_KMAJ>(A, m0, ka, slot_a, offa);
      };
      phase8(std::bool_constant<!kFirst>{}, f1, g1h, f0, g0h, std::integral_constant<int, 0>{}, load_b);
      phase8(std::true_type{}, f0, g0h, f1, g1h, std::integral_constant<int, 2>{}, load_a);
      wait_stages(1);
      stage_barrier();
      sa = next(sa, 2);
      sb = next(sb, 2);
    };
    if (nk > 0) body8(0, std::true_type{}, std::false_type{});
    int64_t j = 1;
    for (; j < fast_end; ++j) body8(j, std::false_type{}, std::true_type{});
    for (; j < nk; ++j) body8(j, std::false_type{}, std::false_type{});
    if (nk > 0) mma8(f1, g1h);  // k-step 1 of the last stage
  }
  wait_stages(0);  // no direct load may still target this workgroup's LDS when it exits
}

// Row (MFMA M index) of accumulator register r in MFMA tile (i, *) for this lane,
// relative to the wave's 128-row range.
__device__ __forceinline__ int acc_row(int i, int r, int lane) { return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---- logits: tile rows = vocabulary, tile cols = chunk tokens -------------------------

struct LogitsArgs {
  Operand w, h;
  int64_t v, vp, rows, C;
  const int64_t* labels;
  float* zy;
  float* pm;
  float* ps;
  bf16_t* prob;  // nullptr: statistics only
  int64_t tiles_m, tiles_n, group_m;
  // recompute mode (backward from the saved LSE): G straight from the logits
  const float* lse_in;    // chunk rows' saved LSE
  const float* grad_out;  // upstream gradient of the loss (device scalar) or nullptr for 1
  const int32_t* nvalid;
  int32_t reduction;
  int64_t ignore_index;
  // fp8 operands: z = h_scale[token] * w_scale[vocabulary row] * (q_h . q_w)
  const float* h_scale;
  const float* w_scale;
  // folded one-pass backward: per-row reference u_t of the stored P, row flags
  const float* uref;
  int32_t* flag;
};

// Recompute-mode epilogue of one wave's 128 vocabulary rows x 128 tokens:
// G = (exp(z - lse) - [j = y]) * scale from the recomputed logits and the
// saved LSE (the backward of the blog's section "2. In-Kernel Gradient
// Computation During the Backward Pass"), scale = upstream gradient times
// 1/n_valid (mean) or 1 (sum), 0 for ignored rows.  G leaves through the
// wave's LDS scratch as whole token rows; the target column's value is
// computed in fp32 and written over its staged slot.
template <bool FULL>
__device__ __forceinline__ void logits_grad_epilogue(const LogitsArgs& a, Acc& acc, int64_t n0, int64_t vbase, int wn,
                                                     int wave, int lane) {
  const int half = lane >> 5;
  const float go = a.grad_out != nullptr ? *a.grad_out : 1.0f;
  const int32_t nv = *a.nvalid;
  const float red = a.reduction == FLCE_SUM ? 1.0f : (nv > 0 ? 1.0f / static_cast<float>(nv) : 0.0f);
  auto in_vocab = [&](int r_row) { return FULL || vbase + r_row < a.v; };
  // The four token columns' labels and LSEs are read before any store: a load
  // issued after a column's stores would wait for them (vmcnt is in order).
  // The loads are unconditional (a row past the end reads the last row and is
  // masked): behind a per-lane branch each would be waited for at its join.
  int64_t labs[4];
  float lses[4];
  static_for<4>([&](auto J) {
    const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
    const int64_t tc = tok < a.rows ? tok : a.rows - 1;
    labs[J] = a.labels[tc];
    lses[J] = a.lse_in[tc];
  });
  static_for<4>([&](auto J) {
    const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
    if (tok >= a.rows) labs[J] = a.ignore_index;
  });
  static_for<4>([&](auto J) {
    const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
    const bool live = tok < a.rows;
    char* stage = reinterpret_cast<char*>(ring()[J]) + kWaveScratchBytes * wave;
    const int64_t lab = labs[J];
    const bool valid = live && lab != a.ignore_index;
    const float sc = valid ? go * red : 0.0f;
    const float l2 = live ? lses[J] * kLog2e : 0.0f;
    const int t = lane & 31;
    static_for<4>([&](auto I) {
      static_for<4>([&](auto Q) {
        float e[4];
        static_for<4>([&](auto U) {
          constexpr int r = Q * 4 + U;
          e[U] = in_vocab(acc_row(I, r, lane)) ? __builtin_amdgcn_exp2f(fmaf(acc.c[I][J][r], kLog2e, -l2)) * sc : 0.0f;
        });
        const int chunk = (I * 4 + Q) ^ (t & 15);
        uint2 pk;
        pk.x = pack_bf16x2(e[0], e[1]);
        pk.y = pack_bf16x2(e[2], e[3]);
        *reinterpret_cast<uint2*>(stage + t * 256 + chunk * 16 + 8 * half) = pk;
      });
    });
    const int64_t q = lab - vbase;
    const int o = static_cast<int>(q & 31);
    if (valid && lab >= 0 && lab < a.v && q >= 0 && q < 128 && ((o >> 2) & 1) == half) {
      const int it = static_cast<int>(q >> 5);
      const int rt = (o >> 3) * 4 + (o & 3);
      float z = 0.0f;
      static_for<4>([&](auto I) {
        static_for<16>([&](auto R) { z = (I == it && R == rt) ? acc.c[I][J][R.value] : z; });
      });
      const float gt = (__builtin_amdgcn_exp2f(fmaf(z, kLog2e, -l2)) - 1.0f) * sc;
      const int qc = static_cast<int>(q);
      *reinterpret_cast<bf16_t*>(stage + t * 256 + (((qc >> 3) ^ (t & 15)) * 16) + (qc & 7) * 2) = f32_to_bf16(gt);
    }
    __builtin_amdgcn_wave_barrier();
    static_for<8>([&](auto Rr) {
      const int tr = 4 * Rr + (lane >> 4), c = lane & 15;
      const uint4 val = *reinterpret_cast<const uint4*>(stage + tr * 256 + ((c ^ (tr & 15)) * 16));
      const int64_t tk = n0 + wn * 128 + J * 32 + tr;
      if (tk < a.rows) *reinterpret_cast<uint4*>(a.prob + tk * a.vp + vbase + 8 * c) = val;
    });
  });
}

// STORE_P: the epilogue also writes P = exp(z - group max) into the chunk buffer
// (a compile-time choice, so that the statistics loop carries no branch).
// FOLD: P = exp(z - r) instead, r = max(u_t, group max - kFoldMargin) with the
// row's reference u_t; a row with r above u_t is flagged.
template <bool RECOMP, bool FP8 = false, bool STORE_P = false, bool FOLD = false>
__global__ __launch_bounds__(kThreads) void mfma_logits_kernel(LogitsArgs a) {
  const int64_t nb = a.tiles_m * a.tiles_n;
  const int64_t t = xcd_remap(blockIdx.x, nb);
  int64_t tm, tn;
  tile_coords(t, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int64_t m0 = tm * TM, n0 = tn * TN;
  Acc acc;
  tile_loop<true, true, FP8>(a.w, a.h, m0, n0, 0, a.w.k_bound, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5;
  const int64_t vbase = m0 + wm * 128;  // this wave's 128-wide vocabulary group
  const int64_t g = vbase / 128;
  if constexpr (FP8) {
    // dequantise: row (I, 4Q + U) of the accumulators is vocabulary row
    // vbase + 32 I + 8 Q + 4 half + U, column J is token n0 + 128 wn + 32 J + lane % 32
    // The group's 128 row scales go through this wave's 8 KB of ring slot 4
    // (the statistics staging below uses slots 0-3): one load per lane, all
    // issued together with the token scales, so nothing waits on them one by
    // one, and the scaling reads them back from LDS without holding registers.
    float sh[4];
    static_for<4>([&](auto J) {
      const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
      sh[J] = a.h_scale[tok < a.rows ? tok : a.rows - 1];
    });
    float* sws = reinterpret_cast<float*>(reinterpret_cast<char*>(ring()[4]) + kWaveScratchBytes * wave);
    {
      const int64_t r = vbase + 2 * lane;  // rows r, r + 1 of the group
      float2 v2;
      if (r + 2 <= a.v) {
        v2 = *reinterpret_cast<const float2*>(a.w_scale + r);
      } else {
        v2.x = r < a.v ? a.w_scale[r < a.v ? r : a.v - 1] : 0.0f;
        v2.y = r + 1 < a.v ? a.w_scale[r + 1 < a.v ? r + 1 : a.v - 1] : 0.0f;
      }
      *reinterpret_cast<float2*>(sws + 2 * lane) = v2;
    }
    static_for<4>([&](auto J) {
      const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
      if (tok >= a.rows) sh[J] = 0.0f;
    });
    __builtin_amdgcn_wave_barrier();
    static_for<4>([&](auto I) {
      static_for<4>([&](auto Q) {
        const float4 q4 = *reinterpret_cast<const float4*>(sws + I * 32 + 8 * Q + 4 * half);
        const float sw[4] = {q4.x, q4.y, q4.z, q4.w};
        static_for<4>([&](auto J) {
          static_for<4>([&](auto U) { acc.c[I][J][Q * 4 + U] *= sw[U] * sh[J]; });
        });
      });
    });
  }
  if constexpr (RECOMP) {
    if (vbase + 128 <= a.v)
      logits_grad_epilogue<true>(a, acc, n0, vbase, wn, wave, lane);
    else
      logits_grad_epilogue<false>(a, acc, n0, vbase, wn, wave, lane);
    return;
  }
  // FULL: every vocabulary row of the group exists (no per-element masks).
  auto epilogue = [&](auto FULL) {
    auto in_vocab = [&](int r_row) { return FULL || vbase + r_row < a.v; };
    // The four token columns' labels are read before any store: a load issued
    // after a column's P stores would wait for them (vmcnt is in order).
    // (unconditional, from a clamped row, so that no branch makes them wait one by one)
    int64_t labs[4];
    float us[4];
    static_for<4>([&](auto J) {
      const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
      labs[J] = a.labels[tok < a.rows ? tok : a.rows - 1];
      if constexpr (FOLD) us[J] = a.uref[tok < a.rows ? tok : a.rows - 1];
    });
    static_for<4>([&](auto J) {
      const int64_t tok = n0 + wn * 128 + J * 32 + (lane & 31);
      const bool live = tok < a.rows;
      char* stage = reinterpret_cast<char*>(ring()[J]) + kWaveScratchBytes * wave;
      // staging row t = token: 16-byte chunk c of the group lands at position c ^ (t % 16)
      const int t = lane & 31;
      char* srow = stage + t * 256 + 8 * half;
      const int sx = t & 15;
      float mx = -INFINITY;
      static_for<4>([&](auto I) {
        static_for<16>([&](auto R) {
          if (in_vocab(acc_row(I, R, lane))) mx = fmaxf(mx, acc.c[I][J][R.value]);
        });
      });
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxl = mx * kLog2e;
      float cref = 1.0f;  // the stored P is e * cref
      if constexpr (FOLD) {
        const float r = fmaxf(us[J], mx - kFoldMargin);
        cref = __builtin_amdgcn_exp2f((mx - r) * kLog2e);
        if (live && half == 0 && vbase < a.v && r != us[J]) a.flag[tok] = 1;
      }
      float s = 0.0f;
      static_for<4>([&](auto I) {
        static_for<4>([&](auto Q) {
          float e[4];
          static_for<4>([&](auto U) {
            constexpr int r = Q * 4 + U;
            e[U] = in_vocab(acc_row(I, r, lane)) ? __builtin_amdgcn_exp2f(fmaf(acc.c[I][J][r], kLog2e, -mxl)) : 0.0f;
            s += e[U];
          });
          if constexpr (STORE_P) {
            uint2 pk;
            pk.x = pack_bf16x2(e[0] * cref, e[1] * cref);
            pk.y = pack_bf16x2(e[2] * cref, e[3] * cref);
            *reinterpret_cast<uint2*>(srow + ((I * 4 + Q) ^ sx) * 16) = pk;
          }
        });
      });
      if constexpr (STORE_P) {
        // The wave's 32 tokens x 128 vocabulary entries of P, 256 bytes per
        // token, go out as four whole token rows per store.
        __builtin_amdgcn_wave_barrier();
        static_for<8>([&](auto Rr) {
          const int tr = 4 * Rr + (lane >> 4), c = lane & 15;
          const uint4 v = *reinterpret_cast<const uint4*>(stage + tr * 256 + ((c ^ (tr & 15)) * 16));
          const int64_t tk = n0 + wn * 128 + J * 32 + tr;
          if (tk < a.rows) *reinterpret_cast<uint4*>(a.prob + tk * a.vp + vbase + 8 * c) = v;
        });
      }
      s += __shfl_xor(s, 32);
      if (live && vbase < a.v) {
        if (half == 0) {
          a.pm[g * a.C + tok] = mx;
          a.ps[g * a.C + tok] = s;
        }
        const int64_t q = labs[J] - vbase;
        const int o = static_cast<int>(q & 31);
        if (q >= 0 && q < 128 && ((o >> 2) & 1) == half) {
          const int it = static_cast<int>(q >> 5);
          const int rt = (o >> 3) * 4 + (o & 3);
          float z = 0.0f;
          static_for<4>([&](auto I) {
            static_for<16>([&](auto R) { z = (I == it && R == rt) ? acc.c[I][J][R.value] : z; });
          });
          a.zy[tok] = z;
        }
      }
    });
  };
  if (vbase + 128 <= a.v)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

// ---- dH: tile rows = chunk tokens, tile cols = hidden; K = vocabulary (split) ----------

struct DhArgs {
  Operand g, w;
  int64_t rows, d;
  int64_t k_split;  // vocabulary columns per split (multiple of TK)
  int64_t tiles_m, tiles_n, splits, group_m;
  bf16_t* out_bf16;  // direct output (splits == 1, bf16)
  float* out_f32;    // direct fp32 output (splits == 1, fp32) or split partials [splits][C][d]
  int64_t part_stride;
  int32_t accumulate;  // splits == 1, fp32 output: add to what out_f32 holds
  const float* rowf;   // FOLD: per-row factor of the output rows
};

template <bool FOLD>
__global__ __launch_bounds__(kThreads) void mfma_dh_kernel(DhArgs a) {
  const int64_t nb = a.tiles_m * a.tiles_n * a.splits;
  const int64_t t = xcd_remap(blockIdx.x, nb);
  const int64_t per_split = a.tiles_n * a.tiles_m;
  const int64_t sp = t / per_split;
  int64_t tm, tn;
  tile_coords(t % per_split, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int64_t m0 = tm * TM, n0 = tn * TN;
  const int64_t k_lo = sp * a.k_split;
  const int64_t k_hi = k_lo + a.k_split < a.g.k_bound ? k_lo + a.k_split : a.g.k_bound;
  Acc acc;
  tile_loop<true, false>(a.g, a.w, m0, n0, k_lo, k_hi, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  static_for<4>([&](auto I) {
    // rows acc_row(I, 4Q + U) = 32 I + 8 Q + 4 (lane / 32) + U: one float4 per Q
    // (the factor array is padded to whole tiles)
    float rf[16];
    if constexpr (FOLD) {
      static_for<4>([&](auto Q) {
        const float4 f4 = *reinterpret_cast<const float4*>(a.rowf + m0 + wm * 128 + I * 32 + 8 * Q + 4 * (lane >> 5));
        rf[4 * Q] = f4.x;
        rf[4 * Q + 1] = f4.y;
        rf[4 * Q + 2] = f4.z;
        rf[4 * Q + 3] = f4.w;
      });
    }
    static_for<4>([&](auto J) {
      const int64_t col = n0 + wn * 128 + J * 32 + (lane & 31);
      static_for<16>([&](auto R) {
        const int64_t row = m0 + wm * 128 + acc_row(I, R, lane);
        if (col < a.d && row < a.rows) {
          float x = acc.c[I][J][R.value];
          if constexpr (FOLD) x *= rf[R.value];
          if (a.out_bf16 != nullptr)
            a.out_bf16[row * a.d + col] = f32_to_bf16(x);
          else if (a.accumulate)
            a.out_f32[row * a.d + col] += x;
          else
            a.out_f32[sp * a.part_stride + row * a.d + col] = x;
        }
      });
    });
  });
}

// dW epilogue of an interior tile.  Between chunks the running sum (hi, lo)
// is kept in a fragment-native order: the two 32x32 subtiles (i, 2p) and
// (i, 2p+1) of a wave store their 32 values per lane inside the very 32x64
// block of the region (dw_out for hi, the workspace for lo) that their
// row-major result covers, as four 1 KB pieces of 8 full 128-byte rows; lane L
// of piece (u, h) holds values 8h .. 8h+7 of subtile 2p+u at row 8(2u+h) + L/8,
// bytes 16 (L % 8).  Each block is read, updated and written by its own wave
// only, so blocks need no synchronisation and the last chunk can overwrite a
// block with the row-major result as soon as it has folded it.
__device__ __forceinline__ uint4* dw_piece(char* block, int64_t row_bytes, int u, int h, uint32_t lane_off) {
  return reinterpret_cast<uint4*>(block + 8 * (2 * u + h) * row_bytes + lane_off);
}

// The running sum is kept exactly, as fp32: hi holds the upper 16 bits of
// each value, lo the lower 16 (byte shuffles, one v_perm_b32 per pair).
__device__ __forceinline__ void split_store(const floatx16& x, uint4* hi0, uint4* hi1, uint4* lo0, uint4* lo1) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t a0 = __float_as_uint(x[2 * k]), a1 = __float_as_uint(x[2 * k + 1]);
    h[k] = (a0 >> 16) | (a1 & 0xffff0000u);
    l[k] = (a0 & 0xffffu) | (a1 << 16);
  }
  *hi0 = make_uint4(h[0], h[1], h[2], h[3]);
  *hi1 = make_uint4(h[4], h[5], h[6], h[7]);
  *lo0 = make_uint4(l[0], l[1], l[2], l[3]);
  *lo1 = make_uint4(l[4], l[5], l[6], l[7]);
}

__device__ __forceinline__ void add_pair(floatx16& x, const uint4& hi0, const uint4& hi1, const uint4& lo0,
                                         const uint4& lo1) {
  const uint32_t h[8] = {hi0.x, hi0.y, hi0.z, hi0.w, hi1.x, hi1.y, hi1.z, hi1.w};
  const uint32_t l[8] = {lo0.x, lo0.y, lo0.z, lo0.w, lo1.x, lo1.y, lo1.z, lo1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] += __uint_as_float((h[k] << 16) | (l[k] & 0xffffu));
    x[2 * k + 1] += __uint_as_float((h[k] & 0xffff0000u) | (l[k] >> 16));
  }
}

// ---- dW: tile rows = vocabulary, tile cols = hidden; K = chunk tokens ----------------

struct DwArgs {
  Operand gt, h;
  int64_t v, d;
  int64_t tiles_m, tiles_n, group_m;
  bf16_t* lo;        // [v][d] lower 16 bits of the fp32 running sum (out holds the upper 16)
  bf16_t* out;       // dw_out
};

template <int MODE>
__device__ __forceinline__ void dw_epilogue_tiled(const DwArgs& a, Acc& acc, int64_t m0, int64_t n0, int wave,
                                                  int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t row_bytes = a.d * static_cast<int64_t>(sizeof(bf16_t));
  const int64_t wave_off = ((m0 + 128 * wm) * a.d + n0 + 128 * wn) * static_cast<int64_t>(sizeof(bf16_t));
  // this wave's private 8 KB of the (now idle) operand ring
  char* scratch = reinterpret_cast<char*>(ring()[0]) + kWaveScratchBytes * wave;
  char* hi_base = reinterpret_cast<char*>(a.out) + wave_off;
  char* lo_base = reinterpret_cast<char*>(a.lo) + wave_off;
  const uint32_t lane_off = static_cast<uint32_t>((lane >> 3) * row_bytes) + static_cast<uint32_t>(lane & 7) * 16u;
  constexpr bool fold = MODE == DW_MID || MODE == DW_LAST;
  constexpr bool keep_split = MODE == DW_FIRST || MODE == DW_MID;
  // block b = (i, p) = (b / 2, b % 2) starts at row 32 i, column 64 p of the wave's quadrant
  auto block_off = [&](int b) { return (32 * (b >> 1)) * row_bytes + 128 * (b & 1); };
  // The stored sums of the next kAhead blocks are in flight while a block is
  // finished.  They travel by direct loads into this wave's 32 KB of the idle
  // operand ring (slot 1 + wave: four 8 KB block buffers of eight 1 KB pieces,
  // lane L's 16 bytes at L * 16), so they hold no registers: register-held
  // prefetches were waited for one load at a time once the accumulators had
  // taken the register file.
  constexpr int kAhead = 3;
  constexpr int kStoresPerBlock = keep_split ? 8 : 4;
  char* fold_lds = reinterpret_cast<char*>(ring()[1 + wave]);
  auto fetch = [&](auto b) {
    char* hb = hi_base + block_off(b);
    char* lb = lo_base + block_off(b);
    char* dst = fold_lds + (b % (kAhead + 1)) * 8192;
    static_for<2>([&](auto u) {
      __builtin_amdgcn_global_load_lds(dw_piece(hb, row_bytes, u, 0, lane_off), FLCE_LDS(dst + (4 * u + 0) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(dw_piece(hb, row_bytes, u, 1, lane_off), FLCE_LDS(dst + (4 * u + 1) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(dw_piece(lb, row_bytes, u, 0, lane_off), FLCE_LDS(dst + (4 * u + 2) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(dw_piece(lb, row_bytes, u, 1, lane_off), FLCE_LDS(dst + (4 * u + 3) * 1024), 16, 0, 0);
    });
  };
  if constexpr (fold) {
    // every wave has waited for its own loads into the ring and finished reading it
    __builtin_amdgcn_s_barrier();
    static_for<kAhead>([&](auto B) { fetch(B); });
  }
  static_for<8>([&](auto B) {
    constexpr int I = B / 2, P = B % 2;
    if constexpr (fold) {
      if constexpr (B + kAhead < 8) fetch(std::integral_constant<int, B + kAhead>{});
      // Memory operations issued after block B's eight loads: the loads of the
      // blocks ahead of it and the result stores of the blocks finished since.
      constexpr int ahead = (B + kAhead < 8 ? B + kAhead : 7) - B;
      constexpr int done = B < kAhead ? B : kAhead;
      wait_vm<8 * ahead + kStoresPerBlock * done>();
      const char* src = fold_lds + (B % (kAhead + 1)) * 8192 + lane * 16;
      static_for<2>([&](auto U) {
        const uint4* q = reinterpret_cast<const uint4*>(src + 4 * U * 1024);
        add_pair(acc.c[I][2 * P + U], q[0], q[64], q[128], q[192]);
      });
    }
    if constexpr (keep_split) {
      char* hb = hi_base + block_off(B);
      char* lb = lo_base + block_off(B);
      static_for<2>([&](auto U) {
        split_store(acc.c[I][2 * P + U], dw_piece(hb, row_bytes, U, 0, lane_off), dw_piece(hb, row_bytes, U, 1, lane_off),
                    dw_piece(lb, row_bytes, U, 0, lane_off), dw_piece(lb, row_bytes, U, 1, lane_off));
      });
    } else {
      // DW_LAST / DW_SINGLE: the block's row-major bf16 result, staged in
      // the wave's LDS scratch so that it leaves as whole 128-byte rows.
      // Neighbouring lanes hold neighbouring columns of the same 16 rows; one
      // swap per row pair gives each lane two columns of one row (a 4-byte
      // LDS write).  Block rows are 128 bytes, their 16-byte chunks XOR-
      // swizzled by the row, so rows r and r+4 use different banks.
      char* blk = scratch + (B & 1) * 4096;
      const int par = lane & 1;
      static_for<2>([&](auto U) {
        constexpr int J = 2 * P + U;
        const int cpair = 32 * U + (lane & 30);  // block column of the pair's even lane
        static_for<8>([&](auto Q) {
          constexpr int R0 = 2 * Q;
          const float x0 = acc.c[I][J][R0], x1 = acc.c[I][J][R0 + 1];
          const float recv =
              __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(par ? x0 : x1), 0xB1, 0xF, 0xF, false));
          const float lo = par ? recv : x0, hi = par ? x1 : recv;  // columns cpair, cpair + 1
          const int rb = 8 * (R0 >> 2) + 4 * (lane >> 5) + (R0 & 3) + par;
          const int chunk = (cpair >> 3) ^ (rb & 7);
          *reinterpret_cast<uint32_t*>(blk + rb * 128 + chunk * 16 + (cpair & 7) * 2) = pack_bf16x2(lo, hi);
        });
      });
      __builtin_amdgcn_wave_barrier();
      // The four row reads are asm so that the compiler does not wait for the
      // direct loads still filling the fold buffers, which it cannot tell apart
      // from this scratch; the asm waits for its own reads only.
      const int c = lane & 7;
      uint32_t ra[4];
      static_for<4>([&](auto Rr) {
        const int rb = 8 * Rr + (lane >> 3);
        ra[Rr] = lds_addr(blk + rb * 128 + ((c ^ (rb & 7)) * 16));
      });
      uint4 v[4];
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
          : "v"(ra[0]), "v"(ra[1]), "v"(ra[2]), "v"(ra[3])
          : "memory");
      static_for<4>([&](auto Rr) {
        const int rb = 8 * Rr + (lane >> 3);
        const int64_t row = m0 + wm * 128 + I * 32 + rb;
        const int64_t col = n0 + wn * 128 + 64 * P + 8 * c;
        *reinterpret_cast<uint4*>(a.out + row * a.d + col) = v[Rr];
      });
    }
  });
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void mfma_dw_kernel(DwArgs a) {
  const int64_t nb = a.tiles_m * a.tiles_n;
  const int64_t t = xcd_remap(blockIdx.x, nb);
  int64_t tm, tn;
  tile_coords(t, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int64_t m0 = tm * TM, n0 = tn * TN;
  Acc acc;
  tile_loop<false, false>(a.gt, a.h, m0, n0, 0, a.gt.k_bound, acc);

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  // The running dW sum across chunks is fp32, split in its upper 16 bits (hi,
  // in dw_out) and lower 16 bits (lo, in the workspace), both inside this
  // tile's own 256x256 region.
  const bool interior = m0 + TM <= a.v && n0 + TN <= a.d;
  if (interior) {
    dw_epilogue_tiled<MODE>(a, acc, m0, n0, wave, lane);
    return;
  }
  // Edge tiles: row-major, element by element.  Per 32x32 subtile a lane
  // owns 16 rows of one column; all loads are issued before any store.
  constexpr bool read_acc = MODE == DW_MID || MODE == DW_LAST;
  constexpr bool keep_split = MODE == DW_FIRST || MODE == DW_MID;
  static_for<4>([&](auto I) {
    static_for<4>([&](auto J) {
      const int64_t col = n0 + wn * 128 + J * 32 + (lane & 31);
      const bool col_ok = col < a.d;
      float prev[16];
      static_for<16>([&](auto R) {
        const int64_t row = m0 + wm * 128 + acc_row(I, R, lane);
        prev[R] = 0.0f;
        if (read_acc && col_ok && row < a.v) {
          const int64_t o = row * a.d + col;
          prev[R] = __uint_as_float((static_cast<uint32_t>(a.out[o]) << 16) | a.lo[o]);
        }
      });
      static_for<16>([&](auto R) {
        const int64_t row = m0 + wm * 128 + acc_row(I, R, lane);
        if (col_ok && row < a.v) {
          const int64_t o = row * a.d + col;
          const float x = acc.c[I][J][R.value] + prev[R];
          if (keep_split) {  // the running sum: x's upper and lower 16 bits
            a.out[o] = static_cast<bf16_t>(__float_as_uint(x) >> 16);
            a.lo[o] = static_cast<bf16_t>(__float_as_uint(x) & 0xffffu);
          } else {
            a.out[o] = f32_to_bf16(x);
          }
        }
      });
    });
  });
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t mfma_logits(const Plan& p, const Work& w, const ChunkArgs& c, int mode, hipStream_t s) {
  LogitsArgs a;
  a.w = Operand{static_cast<const bf16_t*>(c.w), p.d, p.v, p.d};
  a.h = Operand{static_cast<const bf16_t*>(c.h), p.d, c.rows, p.d};
  a.v = p.v;
  a.vp = p.vp;
  a.rows = c.rows;
  a.C = p.chunk;
  a.labels = c.labels;
  a.zy = w.zy;
  a.pm = w.pm;
  a.ps = w.ps;
  a.prob = mode != LOGITS_STATS ? static_cast<bf16_t*>(w.prob) : nullptr;
  a.tiles_m = p.vp / TM;
  a.tiles_n = cdiv(c.rows, TN);
  a.group_m = p.group_m[0];
  a.lse_in = c.lse_in;
  a.grad_out = c.grad_out;
  a.nvalid = w.nvalid;
  a.reduction = c.reduction;
  a.ignore_index = c.ignore_index;
  a.h_scale = c.h_scale;
  a.w_scale = c.w_scale;
  a.uref = w.uref;
  a.flag = w.flag;
  const dim3 grid(static_cast<unsigned>(a.tiles_m * a.tiles_n));
  if (c.fp8) {
    if (mode == LOGITS_PROB) return hipErrorInvalidValue;  // the fp8 path has no one-pass backward
    if (mode == LOGITS_GRAD_FROM_LSE)
      mfma_logits_kernel<true, true><<<grid, kThreads, 0, s>>>(a);
    else
      mfma_logits_kernel<false, true><<<grid, kThreads, 0, s>>>(a);
  } else if (mode == LOGITS_GRAD_FROM_LSE) {
    mfma_logits_kernel<true><<<grid, kThreads, 0, s>>>(a);
  } else if (mode == LOGITS_PROB) {
    if (c.fold)
      mfma_logits_kernel<false, false, true, true><<<grid, kThreads, 0, s>>>(a);
    else
      mfma_logits_kernel<false, false, true><<<grid, kThreads, 0, s>>>(a);
  } else {
    mfma_logits_kernel<false, false, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t mfma_dh(const Plan& p, const Work& w, const ChunkArgs& c, hipStream_t s) {
  DhArgs a;
  a.g = Operand{static_cast<const bf16_t*>(w.prob), p.vp, c.rows, p.vp};
  a.w = Operand{static_cast<const bf16_t*>(c.w), p.d, p.d, p.v};
  a.rows = c.rows;
  a.d = p.d;
  a.splits = p.dh_splits;
  a.k_split = cdiv(cdiv(p.vp, p.dh_splits), TK) * TK;
  a.tiles_m = cdiv(c.rows, TM);
  a.tiles_n = cdiv(p.d, TN);
  a.group_m = p.group_m[1];
  a.part_stride = p.chunk * p.d;
  a.out_bf16 = nullptr;
  a.out_f32 = nullptr;
  a.accumulate = p.dh_splits == 1 && c.dh_accumulate;
  if (p.dh_splits > 1)
    a.out_f32 = w.dhpart;
  else if (p.dtype == FLCE_BF16 && !c.dh_f32)
    a.out_bf16 = static_cast<bf16_t*>(c.dh);
  else
    a.out_f32 = static_cast<float*>(c.dh);
  a.rowf = c.fold ? w.rowf : nullptr;
  const unsigned blocks = static_cast<unsigned>(a.tiles_m * a.tiles_n * a.splits);
  if (c.fold)
    mfma_dh_kernel<true><<<blocks, kThreads, 0, s>>>(a);
  else
    mfma_dh_kernel<false><<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t mfma_dw(const Plan& p, const Work& w, const ChunkArgs& c, hipStream_t s) {
  DwArgs a;
  a.gt = Operand{static_cast<const bf16_t*>(w.prob), p.vp, p.vp, c.rows};
  // folded backward: the token operand is the chunk's bf16(F * H)
  a.h = Operand{static_cast<const bf16_t*>(c.fold ? w.hs : c.h), p.d, p.d, c.rows};
  a.v = p.v;
  a.d = p.d;
  a.tiles_m = p.vp / TM;
  a.tiles_n = cdiv(p.d, TN);
  a.group_m = p.group_m[2];
  a.lo = w.dwlo;
  a.out = static_cast<bf16_t*>(c.dw);
  const dim3 grid(static_cast<unsigned>(a.tiles_m * a.tiles_n));
  switch (c.dw_mode) {
    case DW_FIRST: mfma_dw_kernel<DW_FIRST><<<grid, kThreads, 0, s>>>(a); break;
    case DW_MID: mfma_dw_kernel<DW_MID><<<grid, kThreads, 0, s>>>(a); break;
    case DW_LAST: mfma_dw_kernel<DW_LAST><<<grid, kThreads, 0, s>>>(a); break;
    default: mfma_dw_kernel<DW_SINGLE><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace flce
