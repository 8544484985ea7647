// The ping-pong prefill kernel (prefill_pp_kernel in pa_prefill.hip) in a
// translation unit of its own, so that the build can give it the compiler's
// max-ilp scheduling strategy alone: measured 1.3% faster on the
// Llama-3-8B-shaped chunked prefill, while the same strategy slows the
// four-wave prefill kernel of the shared-prefix pass.
#define PA_PREFILL_PP_TU 1
#include "pa_prefill.hip"
