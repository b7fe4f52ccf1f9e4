// qg_launch.h -- host-side launchers of the libqgemv kernels.  Arguments are
// validated by the C-ABI layer before any of these is called; each returns
// QG_OK or QG_ELAUNCH.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemv.h"
#include "qg_layout.h"

namespace qg {

// Activation rows prepared in a workspace, as the GEMV kernels read them.
struct Prep {
  const int8_t* codes;
  const float* dx;
  const int* nsx;
};
Prep prep_view(const void* ws, const PrepLayout& L);

// A1: quantize rows x [rows][k] into a workspace in the order L (qg_layout.h).
int launch_prepare(const float* x, int rows, int64_t k, void* ws, const PrepLayout& L, hipStream_t s);
// h = x + res, y = RMS norm of h times gamma, A1 of y into ws (prep_layout(rows, k)) when ws is not null.
int launch_add_rmsnorm_prepare(const float* x, const float* res, const float* gamma, float eps, int rows, int64_t k,
                               float* h_out, float* y_out, void* ws, hipStream_t s);
// A1 for up to QG_MAX_SET activation sets (same row count) in one launch.
int launch_prepare_set(const qg_act* acts, int count, int rows, hipStream_t s);
// A1 in the plain layout with code sums (test hook).
int launch_quantize_plain(const float* x, int rows, int64_t k, int8_t* qx, float* dx, int32_t* sx, hipStream_t s);
// Offline weight quantization into a device image.
int launch_quantize_weights(int fmt, const float* w, int64_t n, int64_t k, void* image, hipStream_t s);
// A3 test hook of the pair kernel (3..16 rows): block dots from a pair-order workspace.
int launch_pair_blockdots(int fmt, const void* image, int64_t n, int64_t k, const void* ws, int rows, int32_t* isum,
                          hipStream_t s);
// A3 test hook.
int launch_blockdots(int fmt, const void* image, int64_t n, int64_t k, const int8_t* qx, int rows, int32_t* isum,
                     hipStream_t s);

// One projection of a q8-lane launch.
struct ProjArg {
  const void* image;
  int64_t n, k;
  const void* ws;  // prepared rows (ignored when x is set)
  const float* x;  // fp32 rows, quantized inside the GEMV launch (rows <= 2)
  float* y;        // [rows][n]
};
// Q8_0/Q4_0 GEMV for 1..16 rows over up to QG_MAX_SET projections, one launch.
int launch_qgemv_set(int fmt, const ProjArg* projs, int count, int rows, hipStream_t s);
// Whether `rows` rows of length k are quantized inside the GEMV launch (1-2
// rows whose q8 blocks fit the launch's LDS staging area); otherwise the
// caller quantizes them into the workspace first.
bool fuses_quantization(int fmt, int rows, int64_t k);

// Grouped routed-expert Q8_0 GEMV: the plan launch (which also quantizes the
// x_rows fp32 rows into ws), then the GEMV.
int launch_grouped(const void* images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                   const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, hipStream_t s);
// The grouped plan (workgroup 0): header, sorted, items of at most
// QG_MAX_ROWS assignments of one expert; with x, workgroups 1.. quantize its
// x_rows rows of length k into xprep (A1 rows, or with fp8 the FP8 groups).
int launch_grouped_plan(const int32_t* expert, const int32_t* x_index, int m, int64_t n_experts, int x_rows,
                        int* header, int* sorted, int* items, hipStream_t s, const float* x = nullptr, int64_t k = 0,
                        void* xprep = nullptr, bool fp8 = false);
// FP8 lane, grouped: the plan's items over n x k block-FP8 expert images
// (expert_bytes apart), activation groups of x_rows rows at `ws` (the FP8
// workspace layout), y [m][n].
int launch_grouped_fp8(const void* images, int64_t n, int64_t k, const void* ws, int x_rows, const int* header,
                       const int* sorted, const int* items, const int32_t* x_index, int m, float* y, hipStream_t s,
                       const float* glu = nullptr);
// Whether a grouped FP8 launch of this k can take the SwiGLU of gate/up rows
// in its staging (glu: the rows' FP8 groups kept in LDS).
bool fp8_glu_fits(int64_t k);

// Grouped GEMV on a plan already in `ws` (header, sorted, items at the
// grouped layout's offsets) and rows prepared at `prep` in row order;
// x_index == nullptr: the activation row of assignment a is a.
// max_item_rows: an upper bound on the rows of one work item (the kernel for
// items of more than two rows is launched only when it can have work).
// glu: null, or the fp32 gate/up rows [m][2k] (gate values, then up values)
// whose SwiGLU h = silu(g) * u, quantized in each tile's staging, is the
// activation row of each assignment instead of a prepared row (prep unused);
// requires max_item_rows <= 2 and grouped_glu_fits(k).
int launch_grouped_planned(const void* images, int64_t n_experts, int64_t n, int64_t k, const void* prep, int x_rows,
                           const int* header, const int* sorted, const int* items, const int32_t* x_index, int m,
                           int max_item_rows, float* y, hipStream_t s, const float* glu = nullptr);

// The plan of a routed MoE step as the gate/up launch computes it: from the
// router logits [rows][E] (top-k, a shared expert E when `shared`); the
// launch's workgroup 0 stores it (expert, weight, x_index [rows * slots],
// header, sorted, items).
struct MoeUp {
  const float* logits;
  int rows, E, topk, shared;
  int32_t* expert;
  float* weight;
  int32_t* x_index;
  int* header;
  int* sorted;
  int* items;
  int* dheader;  // the plan's items cut to at most two rows, or null (plan_store)
  int* ditems;
  int plan_off;  // set by the launcher
};
// Rows up to which the gate/up launch of a routed MoE step plans for itself
// (one row a wave of its workgroups) instead of after a plan launch.
constexpr int MOE_UP_PLAN_ROWS = 8;
// The gate/up launch of a routed MoE step: the plan, then the grouped GEMV of
// the (E + shared) n x k images on the input rows prepared at prep (row
// order, rows rows), outputs y [rows * slots][n].
int launch_moe_up(const void* images, int64_t n, int64_t k, const void* prep, const MoeUp& up, float* y,
                  hipStream_t s);
// Whether two SwiGLU rows of length k fit a tile's staging area whole.
bool grouped_glu_fits(int64_t k);
// The down projection of every assignment and the weighted combine in one
// launch (one or two rows; false: the shape needs the grouped launch and the
// combine launch).
bool moe_down_combine_fits(int rows, int slots, int64_t hidden, int64_t ffn);
int launch_moe_down_combine(const void* images, int n_images, int64_t hidden, int64_t ffn, const float* gu,
                            const int32_t* expert, const float* weight, int rows, int slots, float* y, hipStream_t s);

// Fused MoE pieces: routing + plan + input quantization (one workgroup), and
// SwiGLU quantized for the down projection.
// x null: the plan only; fp8: x's FP8 groups into the FP8 workspace xprep
// instead of q8 rows.
int launch_moe_plan(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                    float* weight, int32_t* x_index, int* header, int* sorted, int* items, const float* x, int64_t k,
                    void* xprep, bool fp8, hipStream_t s);
int launch_swiglu_q8(const float* gu, int m, int64_t ffn, void* hprep, hipStream_t s);
// SwiGLU of m gate/up rows into the FP8 workspace of m rows of ffn (ffn % 128 == 0).
int launch_swiglu_fp8(const float* gu, int m, int64_t ffn, void* hws, hipStream_t s);

// f16 lane.
int launch_gemv_f16(const void* image, int64_t n, int64_t k, const float* x, int rows, float* y, hipStream_t s);
// Routed MoE step, first launch: the f16 router GEMV (n < 4096; the bits of
// launch_gemv_f16) into y, beside it the A1 of x into xprep (row order), or
// with fp8 its 1 x 128 FP8 groups (the FP8 workspace layout).
int launch_moe_router(const void* image, int64_t n, int64_t k, const float* x, int rows, float* y, void* xprep,
                      hipStream_t s, bool fp8 = false);
// The FP8 MoE step's gate/up launch planning for itself, as launch_moe_up
// (a row a wave: whether rows fit the launch's waves, moe_up_fp8_fits); xprep
// holds the input rows' FP8 groups.
bool moe_up_fp8_fits(int64_t n, int64_t k, int rows);
int launch_moe_up_fp8(const void* images, int64_t n, int64_t k, const void* xprep, const MoeUp& up, float* y,
                      hipStream_t s);
int launch_f16_pack(const uint16_t* w, int64_t n, int64_t k, void* image, hipStream_t s);
int launch_fp8_quantize_weights(const float* w, int64_t n, int64_t k, void* image, hipStream_t s);
int launch_fp8_prepare(const float* x, int rows, int64_t k, void* ws, hipStream_t s);
int launch_gemv_fp8(const void* image, int64_t n, int64_t k, const void* ws, int rows, float* y, hipStream_t s);

// MoE glue.
int launch_moe_route(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                     int32_t* x_index, float* weight, hipStream_t s);
int launch_swiglu(const float* gu, int m, int64_t ffn, float* h, hipStream_t s);
int launch_moe_combine(const float* o, const float* weight, int rows, int slots, int64_t hidden, float* y,
                       hipStream_t s);

// Device facts, cached per process.
int device_cus();

}  // namespace qg
