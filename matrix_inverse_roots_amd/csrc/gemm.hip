// gemm.hip -- entry point of the batched B x B products on CDNA4 matrix cores (MFMA).
//
// Every solver step of the inverse-root iterations is a product of two B x B blocks, done for all
// N blocks of the stack at once ([PT] Metodologia, item 1: the whole stack goes through batched
// matrix products).  One launch covers one or two batched products (grid = problems x blocks x
// tiles) and fuses the affine combination the iteration needs, D = a*acc + b*C + d*E + g*I, with
// per-block coefficients read on the device (gemm_common.hpp).  The kernels are in gemm_f32.hip
// (fp32 operands), gemm_f16.hip (binary16 or bfloat16 operands, fp32 accumulation) and
// gemm_split.hip (fp32 operands formed on the bfloat16 matrix cores from exact three-piece splits,
// or, in the Clenshaw launches, on the binary16 ones from scaled two-piece splits).
#include <hip/hip_runtime.h>

#include "gemm_common.hpp"

namespace dash {
namespace {

// binary16 products take no C/E operands (their epilogue is built without them)
bool epi_uses_ce(const Product* p, int n) {
  for (int i = 0; i < n; ++i)
    if (p[i].C || p[i].E) return true;
  return false;
}

}  // namespace

hipError_t launch_gemm(const Product* probs, int nprob, int64_t N, int B, dash_prec in_prec, dash_prec out_prec,
                       Trans trans, bool sym, const Epilogue& epi, hipStream_t stream, bool y_sym) {
  if (nprob < 1 || nprob > 2 || N < 1 || B % 64 != 0) return hipErrorInvalidValue;
  gemm::GemmArgs a;
  a.p0 = probs[0];
  a.p1 = nprob > 1 ? probs[1] : probs[0];
  a.nprob = nprob;
  a.N = N;
  a.B = B;
  a.epi = epi;
  // triangle-only products write their mirror straight from the accumulators: no second output
  if (sym && (probs[0].D2 || (nprob > 1 && probs[1].D2))) return hipErrorInvalidValue;
  // folding C into the product needs C == Y in every problem of a triangle-only fp32 NN launch
  // and E in every problem, except the launches that map Y, which have none
  auto fold_ok = [&](const Product& p) { return p.C && p.C == p.Y && (p.map_y ? !p.E : p.E != nullptr); };
  const bool split = in_prec == DASH_FP32_SPLIT || in_prec == DASH_FP32_SPLIT16;
  if (epi.fold_c && !split &&
      (in_prec != DASH_FP32 || !sym || trans != Trans::NN || !fold_ok(probs[0]) || (nprob > 1 && !fold_ok(probs[1]))))
    return hipErrorInvalidValue;
  // operand maps exist in every binary16 kernel and, for the right operand, in the fp32 Clenshaw
  // launches
  const bool maps = probs[0].map_x || probs[0].map_y || (nprob > 1 && (probs[1].map_x || probs[1].map_y));
  const bool map_x = probs[0].map_x || (nprob > 1 && probs[1].map_x);
  // (fp32: every problem of the launch maps its Y)
  if (maps && in_prec == DASH_FP32 && (map_x || !epi.fold_c || (nprob > 1 && probs[0].map_y != probs[1].map_y)))
    return hipErrorInvalidValue;
  // stopped blocks are handled by the fp32 full NN kernel and the binary16 triangle-only kernels
  const bool frz = probs[0].freeze || (nprob > 1 && probs[1].freeze);
  if (frz && (trans != Trans::NN || epi.fold_c || (in_prec == DASH_FP32) == sym)) return hipErrorInvalidValue;
  if (probs[0].pass < 0 || probs[0].pass > 2 || (nprob > 1 && (probs[1].pass < 0 || probs[1].pass > 2)))
    return hipErrorInvalidValue;
  if (in_prec == DASH_FP32) {
    if (out_prec != DASH_FP32) return hipErrorInvalidValue;
    return gemm::launch_f32(a, trans, sym, stream);
  }
  // fp32 operands split into bfloat16 pieces, 256-wide tiles: symmetric results of NN with an
  // exactly symmetric right operand or with C == Y folded, of NT or of TN, or general NN
  // products; no operand maps,
  // stopped blocks or second output.  C is read from memory with its (beta, ib) weight, or, with
  // fold_c (symmetric NN only, C == Y in every problem), enters as (c_over_a coef[ic]) added to
  // X's diagonal: alpha coef[ia] (X + c I) Y
  // two-piece binary16 (DASH_FP32_SPLIT16): the Clenshaw launches (symmetric NN, C == Y folded),
  // general NN products, and symmetric NT / TN products (the statistics), with the magnitude bounds
  // of both operands in every problem
  if (split) {
    const bool h2 = in_prec == DASH_FP32_SPLIT16;
    const bool shape_ok = sym ? (trans != Trans::NN || y_sym || epi.fold_c) : trans == Trans::NN;
    bool fold_ok_split = !epi.fold_c || (sym && trans == Trans::NN);
    for (int i = 0; i < nprob; ++i) {
      if (epi.fold_c && probs[i].C != probs[i].Y) fold_ok_split = false;
      if (h2 && (!probs[i].amax_x || !probs[i].amax_y)) fold_ok_split = false;
    }
    const bool h2_ok = (trans == Trans::NN && sym == epi.fold_c) || (trans != Trans::NN && sym && !epi.fold_c);
    if (out_prec != DASH_FP32 || !shape_ok || maps || frz || !fold_ok_split || probs[0].D2 ||
        (nprob > 1 && probs[1].D2) || B % 256 != 0 || (h2 && !h2_ok))
      return hipErrorInvalidValue;
    return gemm::launch_split(a, sym, trans, y_sym, h2, stream);
  }
  // 2-byte operands (binary16 or bfloat16): output in fp32 or in the operand format
  if ((in_prec != DASH_FP16 && in_prec != DASH_BF16) || (out_prec != DASH_FP32 && out_prec != in_prec))
    return hipErrorInvalidValue;
  if (trans != Trans::NN || epi_uses_ce(probs, nprob)) return hipErrorInvalidValue;
  // binary16-operand products carry no second output
  if (probs[0].D2 || (nprob > 1 && probs[1].D2)) return hipErrorInvalidValue;
  return gemm::launch_f16(a, in_prec, out_prec, sym, y_sym, stream);
}

}  // namespace dash
