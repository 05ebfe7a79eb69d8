// moe_kernels.h -- argument blocks and launchers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- route.hip ----------------------------------------------------------
struct RouteArgs {
    int64_t T;
    int d, E, k;
    float tau;
    const void* x;       // [T, d] bf16 bits or fp32
    const float* Wg;     // [d, E]
    const float* bg;     // [E] or null
    float* logits;       // [T, E] or null (gate kernel: optional output; logits kernel: input)
    int32_t* idx;        // [T, k]
    float* w;            // [T, k]
    int TB, Epad, KC, G;  // launch geometry, from route_config()
    int MR, lkv, lep;     // micro-tile rows, log2(KC / vector), log2(padded E)
};
RouteArgs route_config(int64_t T, int d, int E, int k, float tau, int dtype, int cus);
size_t route_smem_bytes(const RouteArgs& a);
hipError_t launch_route_gate(const RouteArgs& a, int dtype, hipStream_t st);
hipError_t launch_route_logits(const RouteArgs& a, hipStream_t st);
// top-k above the register groups' 32 winners: the selection by rank over
// logits in global memory (any k <= E <= 1024)
constexpr int kRouteGroupMaxK = 32;
hipError_t launch_route_rank(const RouteArgs& a, hipStream_t st);
hipError_t launch_route_variant(const RouteArgs& a, int mode, const float* noise, float scale, float* noisy,
                                hipStream_t st);

// ---- route_mfma.hip (bf16 x, E <= 256): fp32-accurate gate on MFMA ------
bool route_mfma_supported(int dtype, int E, int k);
size_t route_mfma_ws_bytes(int d, int E);   // the three bf16 parts of Wg
hipError_t launch_route_mfma(const RouteArgs& a, uint16_t* W3, int cus, hipStream_t st);

// ---- dispatch.hip -------------------------------------------------------
struct DispatchArgs {
    int64_t T;
    int E, k;
    int64_t cap, max_rows;
    int BT, nblk;          // token block of the histogram / scatter kernels
    const int32_t* idx;    // [T, k]
    int32_t* blkhist;      // [nblk, E] workspace
    int32_t* routed;       // [E] or null
    int32_t* counts;       // [E] or null
    int32_t* offsets;      // [E+1]
    int32_t* perm;         // [max_rows]
    int32_t* slot;         // [T, k]
    float* aux;            // [1] or null
    float lambda;
    // gather
    const void* x;         // [T, d]
    void* x_perm;          // [max_rows, d]
    int64_t row_bytes;     // d * element size
};
int dispatch_block_tokens(int64_t T, int E, int k);
hipError_t launch_hist(const DispatchArgs& a, hipStream_t st);
// the fused bf16 forward's copy: x_pt = the rows of x_perm in the h tile
// layout over h_tiled_rows(max_rows, E) rows of 32 ceil(d/32) columns
// (padding rows and columns zero); perm is padded with -1 as by launch_gather
hipError_t launch_gather_tiled(const DispatchArgs& a, uint16_t* x_pt, int d, hipStream_t st);
// x_perm[slot[t, j]] = x[t] for the kept slots (row-major, row_bytes per row)
hipError_t launch_gather_slots(int64_t T, int k, int64_t max_rows, int64_t row_bytes, const void* x,
                               const int32_t* slot, void* x_perm, hipStream_t st);
hipError_t launch_scatter(const DispatchArgs& a, hipStream_t st);
hipError_t launch_gather(const DispatchArgs& a, hipStream_t st);

// ---- ffn_bf16.hip / ffn_fp32.hip ----------------------------------------
// bf16 pipelined kernel only, for the backward (no bias, [rows, N] row-major):
//   EPI_HGRAD: h = GELU(a) and GELU'(a), both in bf16, to out and out2;
//   EPI_DA: (A B) * out2 (GELU'(a) in bf16, read) in bf16 to out;
//   EPI_WGRAD: out[e] [M, N] fp32 = A[seg(e)]^T B[seg(e)] with A [rows, M] and
//   B [rows, N] row-major (the segments of offsets), zeros for idle experts
enum { EPI_GELU_H = 0, EPI_STORE_F32 = 1, EPI_HGRAD = 2, EPI_DA = 3, EPI_WGRAD = 4 };
struct GemmArgs {
    const void* A;           // [rows, K], row-major, layer dtype
    const void* B;           // [E, K, N], row-major, layer dtype ([E, N, K] for the K-contiguous form)
    const float* bias;       // [E, N], or null for none (bf16 pipelined kernel)
    const int32_t* offsets;  // [E+1] row segments of the experts
    int E, K, N;
    int M;                   // EPI_WGRAD: columns of A (K is the expert's segment)
    void* out;               // EPI_GELU_H: [rows, N] dtype; EPI_STORE_F32: [rows, N] fp32
    // bf16 kernels: the EPI_GELU_H output and the EPI_STORE_F32 input A are h
    // in the tile layout of ffn_bf16.hip (h_tiled_rows rows); fp32 kernels:
    // row-major
    uint16_t* out2;          // GELU'(a) [rows, N] bf16: EPI_HGRAD output, EPI_DA input
};
// rows of the h tile layout for max_rows packed rows over E experts
inline int64_t h_tiled_rows(int64_t max_rows, int64_t E) { return ((max_rows + 15 * E + 15) / 16) * 16; }
// a_tiled (EPI_GELU_H): A is x_perm in the h tile layout (gather_tiled_kernel)
hipError_t launch_ffn_gemm_bf16(const GemmArgs& g, int epi, int64_t max_rows, hipStream_t st, bool a_tiled = false);
// The pipelined 256 x 256 bf16 kernel with explicit operand layouts (the
// backward's expert GEMMs): A row-major (not the h tile layout); B as [E, K, N]
// or, b_kc, [E, N, K] (then K must be a multiple of 32).  max_rows bounds the
// packed rows (EPI_WGRAD: the rows of any one expert's segment).  Returns false
// and launches nothing when the problem is too small for it or outside its
// limits (EPI_WGRAD: max_rows * max(M, N) * 2 >= 2^31, its 32-bit offsets).
bool launch_ffn_gemm_bf16_pipe(const GemmArgs& g, int epi, bool b_kc, int64_t max_rows, hipStream_t st,
                               hipError_t* err);
hipError_t launch_ffn_gemm_f32(const GemmArgs& g, int epi, hipStream_t st);

// ---- combine.hip ----------------------------------------------------------
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st);
hipError_t launch_combine(int64_t T, int d, int k, const float* out_perm, const int32_t* slot,
                          const float* w, float* y, hipStream_t st);
hipError_t launch_aux(int E, int64_t T, int k, float lambda, const int32_t* counts, float* aux,
                      hipStream_t st);

// ---- coact.hip: routing heat map and load telemetry -----------------------
hipError_t launch_coactivation(int64_t T, int k, int E, const int32_t* idx, int32_t* H, int32_t* routed,
                               float* stats, int cus, hipStream_t st);
hipError_t launch_aux_variance(int E, float lambda, const int32_t* load, float* aux, hipStream_t st);

// ---- window_loss.hip: balance loss over a sliding window of calls ---------
size_t window_state_bytes(int64_t E, int64_t W);
hipError_t launch_window_aux(int E, int64_t W, int64_t T, int k, float lambda, const int32_t* counts, void* state,
                             float* aux, float* pbar, hipStream_t st);

// ---- backward.hip: the layer backward ------------------------------------
struct BwGemmArgs {
    const void* A;           // see backward.hip for the three operand patterns
    const void* B;
    int64_t lda, ldb;
    int64_t b_estride;       // elements between experts' weight matrices (NN, NT)
    const int32_t* offsets;  // row segments [E+1]
    int E, M, N, K;
    const float* bias;       // NN recompute: b1 [E, N]
    void* C;                 // output
    void* C2;                // NN: GELU'(a) out; NT with GELU' product: GELU'(a) in
                             // (bf16 in the matrix-core kernel, fp32 in the fp32 one)
};
struct BackwardArgs {
    int64_t T, max_rows;
    int d, E, k, dff;
    float tau;
    const void* x; const float* Wg; const void* W1; const float* b1; const void* W2;
    const float* dy; const int32_t* topk_idx; const float* topk_w; const int32_t* slot;
    const int32_t* offsets; const void* x_perm; const float* out_perm;
    float *dx, *dWg, *dbg, *dW1, *db1, *dW2, *db2;
    // workspace
    float* g;        // [max_rows, d] expert-output gradients (layer dtype; bf16 read through casts)
    void* h;         // [max_rows, dff] recomputed GELU(a), layer dtype
    void* hgrad;     // [max_rows, dff] GELU'(a), layer dtype
    float* da;       // [max_rows, dff] (layer dtype)
    float* dx_perm;  // [max_rows, d]
    float* dw;       // [T, k]
    // gate: the routed (token, expert) pairs grouped by expert (no capacity)
    int BT, nblk;    // dispatch token block and block count
    int32_t* ghist;  // [nblk, E]
    int32_t* goff;   // [E+1]
    int32_t* gperm;  // [T k] token of each grouped row
    int32_t* gslot;  // [T k] grouped row of each (t, j)
    float* dlsel;    // [T, k] gradient of the selected logits
    float* dlr;      // [T k] the same per grouped row
    float* wgt;      // [E, d] Wg transposed
    float* gpart;    // [gate_wgrad_items, d] partial dWg over row chunks
    float* gpartb;   // [gate_wgrad_items] partial dbg
};
// rows of one partial dWg sum; gate_wgrad_items bounds the number of chunks
constexpr int GATE_WGRAD_ROWS = 128;
int64_t gate_wgrad_items(int64_t T, int k, int E);
hipError_t launch_layer_backward(const BackwardArgs& b, int dtype, hipStream_t st);

// device properties (moe_api.hip)
int device_cu_count();

}  // namespace moe
