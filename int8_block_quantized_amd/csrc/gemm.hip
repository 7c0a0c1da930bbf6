// gemm.hip -- block-scaled INT8 GEMM on the gfx950 INT8 matrix cores.
//
// Pages: Jetfire summary, "Approach": linear operators (forward, activation
// gradient and weight gradient) consume INT8 codes with one scale per 32x32
// block and produce INT8 + per-block scales, quantized on-chip.
//
//   C[M x N] = op(A)[M x K] . op(B)[K x N]
//   per output block (I, J), per 32-deep k-block kappa (ascending):
//     P     = exact int32 sum of 32 code products   (one MFMA)
//     sigma = fl(sA[I,kappa] * sB[kappa,J])
//     acc   = fma(sigma, (float)P, acc)              (binary32, VALU)
//   epilogue: store acc (fp32) or requantize the 32x32 block in registers.
//
// One v_mfma_i32_32x32x32_i8 is exactly one (32x32 output block, k-block)
// pair: its K of 32 matches the scale block, so every MFMA result is the
// exact int32 partial that gets rescaled.  The MFMA result is taken in
// architectural VGPRs (built with -amdgpu-mfma-vgpr-form) so the rescale
// costs two VALU instructions per element and k-block (convert, fma) and no
// AGPR reads.  The operands are passed to the MFMA swapped (B fragment
// first) so that a lane owns one output ROW and its 16 accumulators are
// columns 8g + 4h + r (g, r = 0..3, h = lane/32): that layout gives
// 4-column stores and keeps a block's requantization inside one wavefront.
//
// Operand staging.  Tiles go straight from global memory into an S-deep
// ring of LDS stages (global_load_lds_dwordx4; no VGPR round trip), one
// barrier per stage, with the next stages' loads in flight:
//   k-contiguous storage (A with transA=0, B with transB=1): LDS [row][k];
//     fragments are one ds_read_b128 per lane (16 consecutive k);
//   row-contiguous storage (A with transA=1, B with transB=0): LDS keeps the
//     stored [k][row] order; fragments are read with two ds_read_b64_tr_b8
//     (gfx950 transposing LDS read), so the transposition costs no VALU work.
//   Rows are XOR-swizzled in 16-byte chunks so fragment reads are free of
//   bank conflicts.
// A 32x32 block is square, so the transposed operand of the gradients keeps
// its codes and its scale; only the scale-grid index order changes.
//
// Workgroup: GM x GN wavefronts; wavefront tile WM x WN output blocks; LDS
// stages of KB k-blocks in an S-deep ring.  Defaults: 2 x 4 wavefronts of
// 2 x 2 blocks (a 128 x 256 tile), stages of two k-blocks, a two-deep ring,
// the stage's fragments read up front, each MFMA followed by its own rescale
// (PIPE 0), about 125 VGPRs: four wavefronts per SIMD.  The rescale is VALU work (two instructions per
// element and k-block) and the VALU issue rate of one wavefront is far below
// the SIMD's, so occupancy, not MFMA scheduling, sets the pace.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "jf_device.h"
#include "jf_launch.h"
#include "jf_tile_order.h"

#ifndef JF_GEMM_WM
#define JF_GEMM_WM 2
#endif
#ifndef JF_GEMM_WN
#define JF_GEMM_WN 2
#endif
#ifndef JF_GEMM_GM
#define JF_GEMM_GM 2
#endif
#ifndef JF_GEMM_GN
#define JF_GEMM_GN 4
#endif
#ifndef JF_GEMM_KB
#define JF_GEMM_KB 2
#endif
#ifndef JF_GEMM_S
#define JF_GEMM_S 2
#endif
#ifndef JF_GEMM_PIPE
#define JF_GEMM_PIPE 0
#endif
// Partial conversion through the MFMA's C operand (see rescale below).
#ifndef JF_GEMM_BIAS
#define JF_GEMM_BIAS 0
#endif
// 1: every k-block's fragments of a stage are read before its first MFMA;
// 0: k-block kk+1's fragments are read after k-block kk's last MFMA issues.
#ifndef JF_GEMM_FRAG_EARLY
#define JF_GEMM_FRAG_EARLY 1
#endif
// Scale prefetch: the next stage's scales are loaded during this stage.
#ifndef JF_GEMM_SPREF
#define JF_GEMM_SPREF 0
#endif
// Smaller tile for grids that would leave SIMDs with one wavefront or none:
// used when the main tile gives fewer than JF_GEMM_SMALL_BELOW workgroups.
// One 32x32 block per wavefront (64x128 tile, eight wavefronts) quadruples
// the wavefronts of such a grid; with one wavefront per SIMD the per-k-block
// rescale issues about 2.6x slower than with four.
#ifndef JF_GEMM_SMALL_WM
#define JF_GEMM_SMALL_WM 1
#endif
#ifndef JF_GEMM_SMALL_WN
#define JF_GEMM_SMALL_WN 1
#endif
#ifndef JF_GEMM_SMALL_GM
#define JF_GEMM_SMALL_GM 2
#endif
#ifndef JF_GEMM_SMALL_GN
#define JF_GEMM_SMALL_GN 4
#endif
#ifndef JF_GEMM_SMALL_BELOW
#define JF_GEMM_SMALL_BELOW 512
#endif
#ifndef JF_GEMM_WAVES_PER_EU
#define JF_GEMM_WAVES_PER_EU 4
#endif
// Larger tile for the gradient GEMMs' grids that have at least
// JF_GEMM_BIG_MIN tiles of it and at least JF_GEMM_BIG_WORK (tiles x
// k-blocks) of work: 4 x 4 wavefronts of the same 2 x 2 blocks (a 256 x 256
// tile, one workgroup of sixteen wavefronts per CU).  Each MFMA then needs a
// third fewer operand bytes from L2 (256 against 384), and at the power the
// GEMMs draw the GPU's clock rises with less memory traffic (about 2.14
// against 2.05 GHz), which on the activation- and weight-gradient layouts
// outweighs the sixteen-wavefront barrier (+2 to +9% on the hidden-4096
// shapes); on the forward layout (B row-contiguous), on grids of fewer tiles
// and on short contractions (8192 x 4096 x 4096: one workgroup per CU for
// only two tiles' worth of k-blocks) it was 1-5% slower.
#ifndef JF_GEMM_BIG_GM
#define JF_GEMM_BIG_GM 4
#endif
#ifndef JF_GEMM_BIG_GN
#define JF_GEMM_BIG_GN 4
#endif
#ifndef JF_GEMM_BIG_MIN
#define JF_GEMM_BIG_MIN 512
#endif
#ifndef JF_GEMM_BIG_WORK
#define JF_GEMM_BIG_WORK (1 << 17)
#endif

#define JF_GEMM_OCCUPANCY __attribute__((amdgpu_waves_per_eu(JF_GEMM_WAVES_PER_EU)))

namespace jf {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One operand tile of a stage, loaded straight from global memory into LDS
// (global_load_lds_dwordx4: lane i of a wavefront writes 16 bytes at
// LDS base + 16 i, so one instruction fills 1 KiB).  LDS rows are not
// padded; instead the 16-byte chunks of each row are XOR-swizzled so that
// the fragment reads below hit distinct banks.
//   KC = true : k-contiguous operand, LDS [R rows][BK bytes], fragments by
//               ds_read_b128 (16 consecutive k of one row per lane);
//   KC = false: row-contiguous operand, LDS [BK k-rows][R bytes], fragments
//               by two ds_read_b64_tr_b8 (transposing read: in each 16-lane
//               group, lane i receives byte i of the eight 16-byte rows
//               addressed by lane pairs (2j, 2j+1)).
template <int R, int BK, int NW, bool KC>
struct DTile {
    static constexpr int kBytes = R * BK;
    static constexpr int kInstr = kBytes / 1024;       // wavefront loads per stage
    static constexpr int kPerWave = (kInstr + NW - 1) / NW;   // wavefront w issues loads w*kPerWave + j
    // loads issued per stage by wavefront w (fewer, or none, for the last
    // wavefronts when the tile has fewer 1 KiB pieces than the workgroup has
    // wavefronts times kPerWave)
    static __device__ __forceinline__ int loads(int wave) { return max(0, min(kPerWave, kInstr - wave * kPerWave)); }
    static constexpr int CPR = KC ? BK / 16 : R / 16;  // 16-byte chunks per LDS row
    static_assert(CPR == 2 || CPR == 4 || CPR == 8 || CPR == 16, "unsupported tile width");

    // Chunk swizzle of LDS row `row`.  KC: the 16 rows read by one 16-lane
    // pass of ds_read_b128 land in 16 distinct bank groups.  !KC: the eight
    // k-rows x two chunks read by one 32-lane pass of the transposing read do.
    static __device__ __forceinline__ int swz(int row) {
        if constexpr (KC) return CPR == 2 ? (row >> 3) & 1 : CPR == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
        else if constexpr (CPR == 2) return 0;
        else if constexpr (CPR == 4) return ((row >> 2) & 1) << 1;
        else if constexpr (CPR == 8) return ((row >> 1) & 3) << 1;
        else return (row & 7) << 1;
    }

    // Per-lane part of this wavefront's load addresses, the same for every
    // stage: byte offset of the lane's 16 bytes from the stage origin (the
    // stored byte of tile row row0 at the stage's first k).  Rows past the
    // operand's end (nrows) are clamped; their results are discarded.  Off is
    // uint32_t when the offsets are known to fit (NARROW), else int64_t.
    template <typename Off>
    static __device__ __forceinline__ void offsets(int64_t ld, int row0, int nrows, int wave, int lane,
                                                   Off (&off)[kPerWave]) {
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int g = min(wave * kPerWave + j, kInstr - 1) * kWave + lane;   // unused beyond kInstr
            const int lr = g / CPR, c = (g % CPR) ^ swz(g / CPR);
            if constexpr (KC)
                off[j] = (Off)(min(row0 + lr, nrows - 1) - row0) * (Off)ld + (Off)(16 * c);
            else
                off[j] = (Off)lr * (Off)ld + (Off)(min(row0 + 16 * c, nrows - 16) - row0);
        }
    }

    // Stage origin in the stored operand (uniform across the workgroup).
    static __device__ __forceinline__ const int8_t *origin(const int8_t *base, int64_t ld, int row0, int k0) {
        return KC ? base + (int64_t)row0 * ld + k0 : base + (int64_t)k0 * ld + row0;
    }

    // Issue this wavefront's share of one stage's loads.  org: the stage
    // origin; lds_wave: LDS byte address of this wavefront's first 1 KiB of
    // the tile in ring slot 0; OFS: byte offset of the tile's slot.  The
    // loads are inline assembly so that the compiler does not treat every
    // later LDS read as dependent on them (it would wait for all of them,
    // the stages still in flight included); the kernel waits for exactly
    // the stage it consumes instead.  M0 holds each instruction's LDS
    // destination.  NARROW: per-lane offsets fit in 32 bits, so the address
    // is a scalar base plus a VGPR offset.
    template <uint32_t OFS, typename Off>
    static __device__ __forceinline__ void issue(const int8_t *org, const Off (&off)[kPerWave], uint32_t lds_wave,
                                                 int wave) {
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            if (kInstr % kPerWave != 0 || kInstr < NW * kPerWave)
                if (wave * kPerWave + j >= kInstr) break;   // uniform
            const uint32_t dst = lds_wave + OFS + 1024u * j;
            if constexpr (sizeof(Off) == 4) {
                asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :: "v"(off[j]), "s"(org), "{m0}"(dst) : "memory");
            } else {
                asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                             :: "v"(org + off[j]), "{m0}"(dst) : "memory");
            }
        }
    }

    // Fragment of block row `brow` (tile-local) at k-block `kk` of the stage:
    // lane -> row (lane & 31), k = 32 kk + 16 (lane >> 5) + 0..15.
    static __device__ __forceinline__ v4i frag(const int8_t *lds, int brow, int kk, int lane) {
        if constexpr (KC) {
            const int rr = brow * kBlock + (lane & 31), c = 2 * kk + (lane >> 5);
            return *reinterpret_cast<const v4i *>(lds + rr * BK + 16 * (c ^ swz(rr)));
        } else {
            const int g = lane >> 4, m = lane & 15;
            const int kr = kk * kBlock + 16 * (g >> 1) + (m >> 1), c = 2 * brow + (g & 1);
            const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_v2i *)(lds + kr * R + 16 * (c ^ swz(kr)) + 8 * (m & 1)));
            const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_v2i *)(lds + (kr + 8) * R + 16 * (c ^ swz(kr + 8)) + 8 * (m & 1)));
            return v4i{lo.x, lo.y, hi.x, hi.y};
        }
    }
};

// Codes of the 16 values of a lane under one non-zero block scale.  The
// reciprocal-product candidate rne(x * fl(1/s)) is the reference code unless
// x * fl(1/s) lies within 2^-15 of a half-integer (see quant_codes for the
// bound); those values (about 6 in 10^5, or all of them when 1/s overflows)
// are redone with the IEEE quotient, one per lane and pass of a loop whose
// trip count is wave-uniform and almost always zero.  The element is picked
// and put back by selects, so the loop adds no register pressure to the
// main loop's level.
__device__ __forceinline__ void quant_codes_rare(const float (&x)[16], float s, int (&code)[16]) {
    const float r = 1.0f / s;
    const bool finite_r = r < __builtin_inff();
    float n[16];
    uint32_t near = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float t = x[e] * r;
        n[e] = __builtin_rintf(t);
        if (!finite_r || fabsf(t - n[e]) > 0.5f - 0x1p-15f) near |= 1u << e;
    }
    while (__builtin_amdgcn_ballot_w64(near != 0) != 0) {
        if (near != 0) {
            const int k = __builtin_ctz(near);
            near &= near - 1;
            float xk = x[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) xk = k == e ? x[e] : xk;
            const float q = __builtin_rintf(xk / s);
#pragma unroll
            for (int e = 0; e < 16; ++e) n[e] = k == e ? q : n[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) code[e] = (int)__builtin_amdgcn_fmed3f(n[e], -127.0f, 127.0f);   // n is finite
}

template <int WM, int WN, int GM, int GN, int KB, int S, bool A_KC, bool B_KC, bool OUT_I8, bool NARROW>
__global__ __launch_bounds__(64 * GM * GN) JF_GEMM_OCCUPANCY void k_gemm_i8bs(
    const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sA, int64_t ldsa,
    const int8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sB, int64_t ldsb,
    int M, int N, int K, void *__restrict__ Cv, int64_t ldc, float *__restrict__ sC, int tilesN) {
    constexpr int NW = GM * GN;
    constexpr int BM = GM * WM * kBlock, BN = GN * WN * kBlock, BK = KB * kBlock;
    using TA = DTile<BM, BK, NW, A_KC>;
    using TB = DTile<BN, BK, NW, B_KC>;
    constexpr int kStageBytes = TA::kBytes + TB::kBytes;
    constexpr int kMaxLoads = TA::kPerWave + TB::kPerWave;   // vector-memory ops per wave and stage, at most
    // S-deep ring of stages; stage st lives in slot st % S.
    __shared__ __attribute__((aligned(1024))) int8_t lds[S][kStageBytes];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id_uniform();
    const int wr = wave / GN, wc = wave % GN;

    // Tile order: XCD-aware renumbering (jf_tile_order.h).
    const TileCoord tc = tile_of(blockIdx.x, gridDim.x, tilesN);
    const int tm = tc.tm, tn = tc.tn;
    const int row0 = tm * BM, col0 = tn * BN;
    const int nbM = M / kBlock, nbN = N / kBlock, nkb = K / kBlock;
    const int I0 = row0 / kBlock + wr * WM, J0 = col0 / kBlock + wc * WN;

    float acc[WM][WN][16];
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    // K is a multiple of BK (the host picks KB accordingly).
    const int nstage = nkb / KB;
    // Scale pointers of this wave's block rows / columns at the current group
    // of S stages, and the distance between consecutive k-blocks (scale grids
    // have at most 2^30 / 32 entries per row).
    const uint32_t stepA = A_KC ? 1u : (uint32_t)ldsa, stepB = B_KC ? 1u : (uint32_t)ldsb;
    const float *pA[WM], *pB[WN];
#pragma unroll
    for (int a = 0; a < WM; ++a) {
        const int I = min(I0 + a, nbM - 1);
        pA[a] = A_KC ? sA + (int64_t)I * ldsa : sA + I;
    }
#pragma unroll
    for (int b = 0; b < WN; ++b) {
        const int J = min(J0 + b, nbN - 1);
        pB[b] = B_KC ? sB + (int64_t)J * ldsb : sB + J;
    }
    using Off = std::conditional_t<NARROW, uint32_t, int64_t>;
    Off offA[TA::kPerWave], offB[TB::kPerWave];
    TA::offsets(lda, row0, M, wave, lane, offA);
    TB::offsets(ldb, col0, N, wave, lane, offB);
    // LDS address of this wavefront's part of slot 0, and the stored-operand
    // origins of the next stage to load.
    const uint32_t lds_wave = (uint32_t)(uintptr_t)(lds_void *)&lds[0][0] + 1024u * (uint32_t)wave * TA::kPerWave;
    const uint32_t lds_wave_b = (uint32_t)(uintptr_t)(lds_void *)&lds[0][0] + 1024u * (uint32_t)wave * TB::kPerWave;
    const int8_t *nextA = TA::origin(A, lda, row0, 0), *nextB = TB::origin(B, ldb, col0, 0);
    const int nloads = TA::loads(wave) + TB::loads(wave);
    const int64_t strideA = A_KC ? BK : BK * lda, strideB = B_KC ? BK : BK * ldb;
    // Loads of the next stage into ring slot SLOT.  The LDS bases go through
    // an empty asm so the compiler recomputes each M0 value (one scalar add)
    // instead of keeping one register per slot and instruction.
    auto issue = [&](auto slot_c) {
        constexpr uint32_t SLOT = decltype(slot_c)::value;
        uint32_t wa = lds_wave, wb = lds_wave_b;
        asm volatile("" : "+s"(wa), "+s"(wb));
        TA::template issue<SLOT * kStageBytes>(nextA, offA, wa, wave);
        TB::template issue<SLOT * kStageBytes + TA::kBytes>(nextB, offB, wb, wave);
        nextA += strideA;
        nextB += strideB;
    };
    static_for<S - 1>([&](auto p) {
        if (decltype(p)::value < nstage) issue(p);
    });
    // Scales of the current stage, loaded one stage ahead (JF_GEMM_SPREF):
    // the scalar loads are issued after the stage's fragment reads have been
    // waited for, so that wait (lgkmcnt, shared by LDS and scalar loads)
    // never covers a scale load still in flight.
    const float *sA0[WM], *sB0[WN];
#pragma unroll
    for (int a = 0; a < WM; ++a) sA0[a] = pA[a];
#pragma unroll
    for (int b = 0; b < WN; ++b) sB0[b] = pB[b];
    float csa[KB][WM], csb[KB][WN];
    auto load_scales = [&](int stg) {
        const int64_t k0 = (int64_t)min(stg, nstage - 1) * KB;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
#pragma unroll
            for (int a = 0; a < WM; ++a) csa[kk][a] = sA0[a][(k0 + kk) * stepA];
#pragma unroll
            for (int b = 0; b < WN; ++b) csb[kk][b] = sB0[b][(k0 + kk) * stepB];
        }
    };
    if constexpr (JF_GEMM_SPREF) load_scales(0);

    constexpr int NB = WM * WN, T = KB * NB;
    constexpr bool kPipe = JF_GEMM_PIPE;
    constexpr bool kBias = JF_GEMM_BIAS;
    constexpr float kBiasF = 12582912.0f;   // 1.5 * 2^23, bits 0x4B400000
    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = 0x4B400000;
    // One stage; SLOT = st % S is a compile-time constant (the loop below is
    // unrolled by S), so every LDS address is a per-lane base plus an
    // immediate offset.
    auto stage = [&](int st, auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        // This wave's loads of stage st have landed once at most the loads of
        // the stages issued after it are still in flight; the barrier then
        // publishes every wave's part and retires all reads of the slot that
        // is refilled below (read in the previous stage).
        if (S > 2 && st + S - 2 < nstage) {
            // this wavefront's own load count per stage (uniform)
            static_for<kMaxLoads + 1>([&](auto c) {
                if (nloads == decltype(c)::value)
                    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((S - 2) * decltype(c)::value) : "memory");
            });
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        // A bare barrier: __syncthreads() would also drain the loads of the
        // later stages still in flight.
        __builtin_amdgcn_s_barrier();
        const int8_t *la = lds[SLOT];
        const int8_t *lb = la + TA::kBytes;

        // Fragments and scale products.  The scales of k-block st*KB + kk sit
        // at a fixed offset from this group's scale pointers (an immediate
        // when the grid is k-contiguous).
        uint32_t sta = stepA, stb = stepB;      // recomputed per stage, not held per offset
        asm volatile("" : "+s"(sta), "+s"(stb));
        auto load_kk = [&](int kk, v4i (&af)[WM], v4i (&bf)[WN], float (&sg)[WM][WN]) {
            const uint32_t oa = (uint32_t)(SLOT * KB + kk) * sta, ob = (uint32_t)(SLOT * KB + kk) * stb;
            float sa[WM], sb[WN];
#pragma unroll
            for (int a = 0; a < WM; ++a) {
                af[a] = TA::frag(la, wr * WM + a, kk, lane);
                sa[a] = pA[a][oa];
            }
#pragma unroll
            for (int b = 0; b < WN; ++b) {
                bf[b] = TB::frag(lb, wc * WN + b, kk, lane);
                sb[b] = pB[b][ob];
            }
#pragma unroll
            for (int a = 0; a < WM; ++a)
#pragma unroll
                for (int b = 0; b < WN; ++b) sg[a][b] = sa[a] * sb[b];
        };
        // With the bias, the MFMA adds the partial to C = bits of 1.5 * 2^23
        // (integer addition): for |P| < 2^22 the sum's bits are exactly the
        // binary32 number 1.5 * 2^23 + P (same exponent, P added to the
        // significand), and |P| <= 32 * 127^2 = 516128.  Subtracting 1.5 * 2^23
        // is then exact (Sterbenz) and yields (float)P: one add, at twice the
        // issue rate of v_cvt_f32_i32.  Either way the fma gets the same value.
        auto mfma = [&](const v4i &b, const v4i &a) {
            if constexpr (kBias) return __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, bias, 0, 0, 0);
            else return __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, v16i{}, 0, 0, 0);
        };
        auto rescale = [&](float (&acc_b)[16], float sigma, const v16i &p) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pr = p[r];   // (a bit_cast of the vector element itself reads element 0)
                const float pf = kBias ? __int_as_float(pr) - kBiasF : (float)pr;
                acc_b[r] = __builtin_fmaf(sigma, pf, acc_b[r]);
            }
        };
        if constexpr (kPipe) {
            v4i af[KB][WM], bf[KB][WN];
            float sg[KB][WM][WN];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) load_kk(kk, af[kk], bf[kk], sg[kk]);
            // Refill the slot read by stage st-1 with stage st+S-1.
            if (st + S - 1 < nstage) issue(std::integral_constant<int, (SLOT + S - 1) % S>{});
            // Software pipeline over the stage's (k-block, output block)
            // pairs: the MFMA of pair t+1 is issued before the rescale of
            // pair t, so the matrix core works while the VALU converts and
            // accumulates.
            v16i pc = mfma(bf[0][0], af[0][0]);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int kk = t / NB, a = (t % NB) / WN, b = t % WN;
                v16i pn;
                if (t + 1 < T) {
                    const int kn = (t + 1) / NB, an = ((t + 1) % NB) / WN, bn = (t + 1) % WN;
                    pn = mfma(bf[kn][bn], af[kn][an]);
                }
                // the next MFMA stays ahead of this rescale in the schedule
                __builtin_amdgcn_sched_barrier(0);
                rescale(acc[a][b], sg[kk][a][b], pc);
                __builtin_amdgcn_sched_barrier(0);
                if (t + 1 < T) pc = pn;
            }
        } else if constexpr (JF_GEMM_FRAG_EARLY && JF_GEMM_SPREF) {
            // Scale products from the prefetched scales first (their loads
            // were issued a stage ago), then every fragment of the stage.
            float sg[KB][WM][WN];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int a = 0; a < WM; ++a)
#pragma unroll
                    for (int b = 0; b < WN; ++b) sg[kk][a][b] = csa[kk][a] * csb[kk][b];
            __builtin_amdgcn_sched_barrier(0);
            v4i af[KB][WM], bf[KB][WN];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
#pragma unroll
                for (int a = 0; a < WM; ++a) af[kk][a] = TA::frag(la, wr * WM + a, kk, lane);
#pragma unroll
                for (int b = 0; b < WN; ++b) bf[kk][b] = TB::frag(lb, wc * WN + b, kk, lane);
            }
            if (st + S - 1 < nstage) issue(std::integral_constant<int, (SLOT + S - 1) % S>{});
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int a = 0; a < WM; ++a)
#pragma unroll
                    for (int b = 0; b < WN; ++b) {
                        const v16i p = mfma(bf[kk][b], af[kk][a]);
                        rescale(acc[a][b], sg[kk][a][b], p);
                        __builtin_amdgcn_sched_barrier(0);
                        if (kk == 0 && a == 0 && b == 0) {
                            // every fragment read of the stage has been waited
                            // for by now (the first MFMA needed them)
                            load_scales(st + 1);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
        } else if constexpr (JF_GEMM_FRAG_EARLY) {
            // Every k-block's fragments and scale products of the stage are
            // read first (the later k-blocks' LDS reads overlap the first
            // k-block's MFMAs), then each MFMA is followed by its rescale.
            v4i af[KB][WM], bf[KB][WN];
            float sg[KB][WM][WN];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) load_kk(kk, af[kk], bf[kk], sg[kk]);
            if (st + S - 1 < nstage) issue(std::integral_constant<int, (SLOT + S - 1) % S>{});
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int a = 0; a < WM; ++a)
#pragma unroll
                    for (int b = 0; b < WN; ++b) {
                        const v16i p = mfma(bf[kk][b], af[kk][a]);
                        rescale(acc[a][b], sg[kk][a][b], p);
                        __builtin_amdgcn_sched_barrier(0);
                    }
        } else {
            // One k-block's fragments at a time: those of k-block kk+1 are
            // read into the same registers once k-block kk's last MFMA has
            // taken its operands, and arrive during that MFMA's rescale.
            v4i af[WM], bf[WN];
            float sg[WM][WN];
            load_kk(0, af, bf, sg);
            if (st + S - 1 < nstage) issue(std::integral_constant<int, (SLOT + S - 1) % S>{});
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int a = 0; a < WM; ++a)
#pragma unroll
                    for (int b = 0; b < WN; ++b) {
                        const v16i p = mfma(bf[b], af[a]);
                        const float sigma = sg[a][b];
                        if (a == WM - 1 && b == WN - 1 && kk + 1 < KB) {
                            float sg_n[WM][WN];
                            load_kk(kk + 1, af, bf, sg_n);
#pragma unroll
                            for (int i = 0; i < WM; ++i)
#pragma unroll
                                for (int j = 0; j < WN; ++j) sg[i][j] = sg_n[i][j];
                        }
                        rescale(acc[a][b], sigma, p);
                        __builtin_amdgcn_sched_barrier(0);
                    }
        }
    };
    for (int st0 = 0; st0 < nstage; st0 += S) {
        static_for<S>([&](auto u) {
            if (st0 + decltype(u)::value < nstage) stage(st0 + decltype(u)::value, u);
        });
#pragma unroll
        for (int a = 0; a < WM; ++a) pA[a] += (int64_t)S * KB * stepA;
#pragma unroll
        for (int b = 0; b < WN; ++b) pB[b] += (int64_t)S * KB * stepB;
    }

    // Epilogue.  Lane owns row 32I + (lane & 31); accumulator r is column
    // 8(r/4) + 4(lane/32) + r%4 of block J.
    const int frow = lane & 31, hc = 4 * (lane >> 5);
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            // one block at a time: interleaving the blocks' reductions would
            // raise the register count above the main loop's
            __builtin_amdgcn_sched_barrier(0);
            const int I = I0 + a, J = J0 + b;
            if (I >= nbM || J >= nbN) continue;
            const int64_t row = (int64_t)I * kBlock + frow;
            const int64_t col = (int64_t)J * kBlock + hc;
            if constexpr (OUT_I8) {
                float m = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[a][b][r]));
                m = wave_max_nonneg(m);
                const float sc = block_scale(m);
                int code[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) code[r] = 0;
                if (sc != 0.0f) quant_codes_rare(acc[a][b], sc, code);
                int8_t *C = reinterpret_cast<int8_t *>(Cv);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<uint32_t *>(C + row * ldc + col + 8 * g) =
                        pack4(code[4 * g], code[4 * g + 1], code[4 * g + 2], code[4 * g + 3]);
                if (lane == 0) sC[(int64_t)I * nbN + J] = sc;
            } else {
                float *C = reinterpret_cast<float *>(Cv);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4 *>(C + row * ldc + col + 8 * g) =
                        f32x4{acc[a][b][4 * g + 0], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
            }
        }
}

template <int WM, int WN, int GM, int GN, int KB, int S, bool A_KC, bool B_KC, bool OUT_I8, bool NARROW>
hipError_t launch_cfg(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const float *sA,
                      const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc, float *sC,
                      hipStream_t stream) {
    constexpr int BM = GM * WM * kBlock, BN = GN * WN * kBlock;
    const int64_t tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
    const int64_t ldsa = A_KC ? K / kBlock : M / kBlock;
    const int64_t ldsb = B_KC ? K / kBlock : N / kBlock;
    hipLaunchKernelGGL((k_gemm_i8bs<WM, WN, GM, GN, KB, S, A_KC, B_KC, OUT_I8, NARROW>), dim3((unsigned)(tilesM * tilesN)),
                       dim3(64 * GM * GN), 0, stream, A, lda, sA, ldsa, B, ldb, sB, ldsb, (int)M, (int)N, (int)K, C,
                       ldc, sC, (int)tilesN);
    return hipGetLastError();
}

template <int WM, int WN, int GM, int GN, int KB, int S, bool A_KC, bool B_KC, bool OUT_I8>
hipError_t dispatch_narrow(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const float *sA,
                           const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc, float *sC,
                           hipStream_t stream) {
    // Per-lane load offsets stay below (tile edge) * ld + tile edge; below
    // 2^31 they go in one 32-bit VGPR beside a scalar base.
    constexpr int64_t kEdge = std::max({GM * WM * kBlock, GN * WN * kBlock, KB * kBlock});
    const bool narrow = (lda + 1) * kEdge < (int64_t(1) << 31) && (ldb + 1) * kEdge < (int64_t(1) << 31);
    if (narrow)
        return launch_cfg<WM, WN, GM, GN, KB, S, A_KC, B_KC, OUT_I8, true>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc,
                                                                           sC, stream);
    return launch_cfg<WM, WN, GM, GN, KB, S, A_KC, B_KC, OUT_I8, false>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC,
                                                                        stream);
}

template <bool A_KC, bool B_KC, bool OUT_I8>
hipError_t dispatch_kb(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const float *sA,
                       const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc, float *sC,
                       hipStream_t stream) {
    // Stage shape: two k-blocks per stage (64-byte row segments per load;
    // 32-byte ones load much worse when an operand is k-contiguous) in a
    // two-deep ring, which leaves LDS for four wavefronts per SIMD.  A stage
    // must lie inside K; odd K/32 falls back to one k-block per stage.
    // Tile: the 256 x 256 one for the gradient layouts when the grid has at
    // least JF_GEMM_BIG_MIN of them, else the 128 x 256 main tile; grids of fewer than
    // JF_GEMM_SMALL_BELOW main tiles take the smaller tile (the per-element
    // k order, and so every result bit, is the same for all three).
    if ((K / kBlock) % JF_GEMM_KB != 0)
        return dispatch_narrow<JF_GEMM_WM, JF_GEMM_WN, 2, 2, 1, 4, A_KC, B_KC, OUT_I8>(M, N, K, A, lda, sA, B, ldb,
                                                                                 sB, C, ldc, sC, stream);
    constexpr int64_t GBM = JF_GEMM_BIG_GM * JF_GEMM_WM * kBlock, GBN = JF_GEMM_BIG_GN * JF_GEMM_WN * kBlock;
    if constexpr (!(A_KC && !B_KC)) {   // not the forward layout
        const int64_t big = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
        if (JF_GEMM_BIG_MIN > 0 && big >= JF_GEMM_BIG_MIN && big * (K / kBlock) >= JF_GEMM_BIG_WORK)
            return dispatch_narrow<JF_GEMM_WM, JF_GEMM_WN, JF_GEMM_BIG_GM, JF_GEMM_BIG_GN, JF_GEMM_KB, JF_GEMM_S,
                                   A_KC, B_KC, OUT_I8>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    }
    constexpr int64_t BM = JF_GEMM_GM * JF_GEMM_WM * kBlock, BN = JF_GEMM_GN * JF_GEMM_WN * kBlock;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tiles < JF_GEMM_SMALL_BELOW)
        return dispatch_narrow<JF_GEMM_SMALL_WM, JF_GEMM_SMALL_WN, JF_GEMM_SMALL_GM, JF_GEMM_SMALL_GN, JF_GEMM_KB,
                               JF_GEMM_S, A_KC, B_KC, OUT_I8>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    return dispatch_narrow<JF_GEMM_WM, JF_GEMM_WN, JF_GEMM_GM, JF_GEMM_GN, JF_GEMM_KB, JF_GEMM_S, A_KC, B_KC, OUT_I8>(
        M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
}

template <bool A_KC, bool B_KC>
hipError_t dispatch_out(bool out_i8, int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                        const float *sA, const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc,
                        float *sC, hipStream_t stream) {
    if (out_i8) return dispatch_kb<A_KC, B_KC, true>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    return dispatch_kb<A_KC, B_KC, false>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
}

}  // namespace

hipError_t launch_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                       const float *sA, const int8_t *B, int64_t ldb, const float *sB, bool out_i8, void *C,
                       int64_t ldc, float *sC, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    // A is k-contiguous when stored M x K (transA = 0); B when stored N x K (transB = 1).
    const bool akc = transA == 0, bkc = transB == 1;
    if (akc && bkc) return dispatch_out<true, true>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    if (akc && !bkc) return dispatch_out<true, false>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    if (!akc && bkc) return dispatch_out<false, true>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    return dispatch_out<false, false>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
}

}  // namespace jf
