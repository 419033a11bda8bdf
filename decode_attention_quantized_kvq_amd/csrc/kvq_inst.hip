// kvq_inst.hip -- one family of the split kernel's instances (key width,
// value width, paged storage, zero point), selected at compile time by
// KVQ_KB, KVQ_VB, KVQ_PG and KVQ_ZP, so that the families compile in
// parallel; kvq.hip declares them all.
#include <hip/hip_runtime.h>

#include "kvq_decode_quant.hpp"

#if !defined(KVQ_KB) || !defined(KVQ_VB) || !defined(KVQ_PG) || !defined(KVQ_ZP)
#error "compile with -DKVQ_KB=.. -DKVQ_VB=.. -DKVQ_PG=.. -DKVQ_ZP=.."
#endif

namespace kvq {
KVQ_QUANT_FAMILY(KVQ_QUANT_DEFINE, KVQ_KB, KVQ_VB, KVQ_PG, KVQ_ZP)
}
