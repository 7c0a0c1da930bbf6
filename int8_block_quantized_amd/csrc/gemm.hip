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
// Operand staging.  Tiles go global -> registers (16-byte loads along the
// stored rows, so every load is coalesced) -> LDS, double-buffered:
//   k-contiguous storage (A with transA=0, B with transB=1): LDS [row][k];
//     fragments are one ds_read_b128 per lane (16 consecutive k);
//   row-contiguous storage (A with transA=1, B with transB=0): LDS keeps the
//     stored [k][row] order; fragments are read with two ds_read_b64_tr_b8
//     (gfx950 transposing LDS read: in each 16-lane group, lane i receives
//     byte i of the eight 16-byte rows addressed by lane pairs (2j, 2j+1)),
//     so the transposition costs no VALU work.
// A 32x32 block is square, so the transposed operand of the gradients keeps
// its codes and its scale; only the scale-grid index order changes.
//
// Workgroup: GM x GN wavefronts; wavefront tile WM x WN output blocks; LDS
// stages of KB k-blocks.  Row pitches are padded so fragment reads are free
// of bank conflicts.
#include "jf_device.h"
#include "jf_launch.h"

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
#define JF_GEMM_GN 2
#endif
#ifndef JF_GEMM_KB
#define JF_GEMM_KB 2
#endif

namespace jf {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// Tile of a k-contiguous operand: R logical rows x BK k-bytes, LDS [row][k].
template <int R, int BK, int NT>
struct TileK {
    static constexpr int P = BK + 16;                  // row pitch: conflict-free b128 reads
    static constexpr int kBytes = R * P;
    static constexpr int kPer = R * BK / 16 / NT;      // 16-byte pieces per thread
    static_assert(R * BK / 16 % NT == 0, "tile must split evenly over the workgroup");
    u32x4 reg[kPer];

    // base/ld: stored operand; row0: first logical row of the tile; nrows:
    // logical rows of the operand; k0: first k of the stage; K: total k.
    __device__ __forceinline__ void load(const int8_t *__restrict__ base, int64_t ld, int row0, int nrows, int k0,
                                         int K, int tid) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int c = tid + NT * p;
            const int r = c / (BK / 16), kc = c % (BK / 16);
            const int grow = min(row0 + r, nrows - 1);
            const int k = k0 + 16 * kc;
            reg[p] = k < K ? *reinterpret_cast<const u32x4 *>(base + (int64_t)grow * ld + k) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(int8_t *__restrict__ lds, int tid) const {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int c = tid + NT * p;
            const int r = c / (BK / 16), kc = c % (BK / 16);
            *reinterpret_cast<u32x4 *>(lds + r * P + 16 * kc) = reg[p];
        }
    }
    // Fragment of block row `brow` (tile-local) at k-block `kk` of the stage:
    // lane -> row (lane & 31), k = 32 kk + 16 (lane >> 5) + 0..15.
    static __device__ __forceinline__ v4i frag(const int8_t *lds, int brow, int kk, int lane) {
        return *reinterpret_cast<const v4i *>(lds + (brow * kBlock + (lane & 31)) * P + kk * kBlock +
                                              16 * (lane >> 5));
    }
};

// Tile of a row-contiguous operand: BK k-rows x R logical rows, LDS [k][row].
template <int R, int BK, int NT>
struct TileT {
    static constexpr int P = R + 32;                   // row pitch: conflict-free tr8 reads
    static constexpr int kBytes = BK * P;
    static constexpr int kPer = BK * R / 16 / NT;
    static_assert(BK * R / 16 % NT == 0, "tile must split evenly over the workgroup");
    u32x4 reg[kPer];

    __device__ __forceinline__ void load(const int8_t *__restrict__ base, int64_t ld, int row0, int nrows, int k0,
                                         int K, int tid) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int c = tid + NT * p;
            const int k = c / (R / 16), ic = c % (R / 16);
            const int gcol = min(row0 + 16 * ic, nrows - 16);
            const int kr = k0 + k;
            reg[p] = kr < K ? *reinterpret_cast<const u32x4 *>(base + (int64_t)kr * ld + gcol) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(int8_t *__restrict__ lds, int tid) const {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int c = tid + NT * p;
            const int k = c / (R / 16), ic = c % (R / 16);
            *reinterpret_cast<u32x4 *>(lds + k * P + 16 * ic) = reg[p];
        }
    }
    // Same fragment as TileK::frag, gathered from the [k][row] layout: two
    // transposing reads of 8 k-rows each.  In 16-lane group g, lane pair
    // (2j, 2j+1) addresses k-row 16 (g/2) + j, columns 16 (g%2) .. +15.
    static __device__ __forceinline__ v4i frag(const int8_t *lds, int brow, int kk, int lane) {
        const int g = lane >> 4, m = lane & 15;
        const int off = (kk * kBlock + 16 * (g >> 1) + (m >> 1)) * P + brow * kBlock + 16 * (g & 1) + 8 * (m & 1);
        const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(lds + off));
        const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(lds + off + 8 * P));
        return v4i{lo.x, lo.y, hi.x, hi.y};
    }
};

template <bool KC, int R, int BK, int NT>
using TileOf = typename std::conditional<KC, TileK<R, BK, NT>, TileT<R, BK, NT>>::type;

template <int WM, int WN, int GM, int GN, int KB, bool A_KC, bool B_KC, bool OUT_I8>
__global__ __launch_bounds__(64 * GM * GN) void k_gemm_i8bs(
    const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sA, int64_t ldsa,
    const int8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sB, int64_t ldsb,
    int M, int N, int K, void *__restrict__ Cv, int64_t ldc, float *__restrict__ sC, int tilesN) {
    constexpr int NT = 64 * GM * GN;
    constexpr int BM = GM * WM * kBlock, BN = GN * WN * kBlock, BK = KB * kBlock;
    using TA = TileOf<A_KC, BM, BK, NT>;
    using TB = TileOf<B_KC, BN, BK, NT>;
    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][TA::kBytes];
    __shared__ __attribute__((aligned(16))) int8_t lds_b[2][TB::kBytes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id_uniform();
    const int wr = wave / GN, wc = wave % GN;

    const int tm = blockIdx.x / tilesN, tn = blockIdx.x - tm * tilesN;
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

    const int nstage = (nkb + KB - 1) / KB;
    TA ta;
    TB tb;
    if (nstage > 0) {
        ta.load(A, lda, row0, M, 0, K, tid);
        tb.load(B, ldb, col0, N, 0, K, tid);
        ta.store(lds_a[0], tid);
        tb.store(lds_b[0], tid);
    }
    __syncthreads();

    constexpr int NB = WM * WN, T = KB * NB;
    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nstage;
        if (more) {
            ta.load(A, lda, row0, M, (st + 1) * BK, K, tid);
            tb.load(B, ldb, col0, N, (st + 1) * BK, K, tid);
        }
        // Fragments and scale products of the whole stage.  k-blocks past K
        // (last stage of a K that is not a multiple of BK) were zero-filled,
        // so their partial is exactly 0 and fma(sigma, 0, acc) leaves acc
        // unchanged (acc is never -0); their scale index is clamped in range.
        v4i af[KB][WM], bf[KB][WN];
        float sg[KB][WM][WN];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int kb = min(st * KB + kk, nkb - 1);
            float sa[WM], sb[WN];
#pragma unroll
            for (int a = 0; a < WM; ++a) {
                af[kk][a] = TA::frag(lds_a[buf], wr * WM + a, kk, lane);
                const int I = min(I0 + a, nbM - 1);
                sa[a] = A_KC ? sA[(int64_t)I * ldsa + kb] : sA[(int64_t)kb * ldsa + I];
            }
#pragma unroll
            for (int b = 0; b < WN; ++b) {
                bf[kk][b] = TB::frag(lds_b[buf], wc * WN + b, kk, lane);
                const int J = min(J0 + b, nbN - 1);
                sb[b] = B_KC ? sB[(int64_t)J * ldsb + kb] : sB[(int64_t)kb * ldsb + J];
            }
#pragma unroll
            for (int a = 0; a < WM; ++a)
#pragma unroll
                for (int b = 0; b < WN; ++b) sg[kk][a][b] = sa[a] * sb[b];
        }
        // Software pipeline over the stage's (k-block, output block) pairs:
        // the MFMA of pair t+1 is issued before the rescale of pair t, so the
        // matrix core works while the VALU converts and accumulates.
        v16i pc = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[0][0], af[0][0], v16i{}, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int kk = t / NB, a = (t % NB) / WN, b = t % WN;
            float sigma = sg[kk][a][b];
            v16i pn;
            if (t + 1 < T) {
                const int kn = (t + 1) / NB, an = ((t + 1) % NB) / WN, bn = (t + 1) % WN;
                pn = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[kn][bn], af[kn][an], v16i{}, 0, 0, 0);
                // keeps the next MFMA ahead of this rescale in the schedule
                asm volatile("; mfma before rescale" : "+v"(sigma) : "v"(pn));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = __builtin_fmaf(sigma, (float)pc[r], acc[a][b][r]);
            if (t + 1 < T) pc = pn;
        }
        if (more) {
            // Fence: the next stage's LDS writes wait on its global loads, so
            // they must not be hoisted above this stage's rescale work.
            __builtin_amdgcn_sched_barrier(0);
            ta.store(lds_a[buf ^ 1], tid);
            tb.store(lds_b[buf ^ 1], tid);
        }
        __syncthreads();
    }

    // Epilogue.  Lane owns row 32I + (lane & 31); accumulator r is column
    // 8(r/4) + 4(lane/32) + r%4 of block J.
    const int frow = lane & 31, hc = 4 * (lane >> 5);
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            const int I = I0 + a, J = J0 + b;
            if (I >= nbM || J >= nbN) continue;
            const int64_t row = (int64_t)I * kBlock + frow;
            const int64_t col = (int64_t)J * kBlock + hc;
            if constexpr (OUT_I8) {
                float m = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[a][b][r]));
                m = wave_max(m);
                const float sc = block_scale(m);
                int8_t *C = reinterpret_cast<int8_t *>(Cv);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t w = 0;
                    if (sc != 0.0f)
                        w = pack4(quant_code(acc[a][b][4 * g + 0], sc), quant_code(acc[a][b][4 * g + 1], sc),
                                  quant_code(acc[a][b][4 * g + 2], sc), quant_code(acc[a][b][4 * g + 3], sc));
                    *reinterpret_cast<uint32_t *>(C + row * ldc + col + 8 * g) = w;
                }
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

template <int WM, int WN, int GM, int GN, int KB, bool A_KC, bool B_KC, bool OUT_I8>
hipError_t launch_cfg(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const float *sA,
                      const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc, float *sC,
                      hipStream_t stream) {
    constexpr int BM = GM * WM * kBlock, BN = GN * WN * kBlock;
    const int64_t tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
    const int64_t ldsa = A_KC ? K / kBlock : M / kBlock;
    const int64_t ldsb = B_KC ? K / kBlock : N / kBlock;
    hipLaunchKernelGGL((k_gemm_i8bs<WM, WN, GM, GN, KB, A_KC, B_KC, OUT_I8>), dim3((unsigned)(tilesM * tilesN)),
                       dim3(64 * GM * GN), 0, stream, A, lda, sA, ldsa, B, ldb, sB, ldsb, (int)M, (int)N, (int)K, C,
                       ldc, sC, (int)tilesN);
    return hipGetLastError();
}

template <bool A_KC, bool B_KC>
hipError_t dispatch_out(bool out_i8, int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                        const float *sA, const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc,
                        float *sC, hipStream_t stream) {
    constexpr int WM = JF_GEMM_WM, WN = JF_GEMM_WN, GM = JF_GEMM_GM, GN = JF_GEMM_GN, KB = JF_GEMM_KB;
    if (out_i8)
        return launch_cfg<WM, WN, GM, GN, KB, A_KC, B_KC, true>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    return launch_cfg<WM, WN, GM, GN, KB, A_KC, B_KC, false>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
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
