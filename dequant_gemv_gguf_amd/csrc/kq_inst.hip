// kq_inst.hip -- one object of the library's launchers: those of the format
// with type id KQ_INST_TYPE, or the mixed launcher of the pair of K-quant
// formats KQ_INST_A < KQ_INST_B.  The build compiles this file once per format
// and once per pair, in parallel.
#include "kq_impl.h"

namespace kq {
#if defined(KQ_INST_TYPE)
KQ_TYPE_LAUNCHERS(template, KQ_INST_TYPE)
#elif defined(KQ_INST_A) && defined(KQ_INST_B)
KQ_MIXED_LAUNCHER(template, KQ_INST_A, KQ_INST_B)
#else
#error "define KQ_INST_TYPE, or KQ_INST_A and KQ_INST_B"
#endif
} // namespace kq
