// Status strings and version of the tree-verification library.
#include "tv_common.h"

extern "C" const char* tv_status_string(int code) {
  switch (code) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_SHAPE: return "a size or stride is out of range";
    case TV_ERR_DTYPE: return "unknown element type";
    case TV_ERR_ALIGN: return "pointer or stride misaligned";
    case TV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TV_ERR_UNSUPPORTED: return "unsupported configuration";
    case TV_ERR_HIP: return "HIP runtime error";
    case TV_ROW_BAD_PARENT: return "row: a parent link is not a smaller node index";
    case TV_ROW_CTX_BOUND: return "row: context length outside its bounds";
    case TV_ROW_NNODES: return "row: n_nodes outside [0, T]";
    case TV_ROW_BAD_TOKEN: return "row: a draft token is outside the vocabulary";
    case TV_ROW_BAD_PATH: return "row: the accepted path is not an increasing walk from the root";
    case TV_ROW_BAD_START: return "row: packed rows outside [0, rows_total)";
    default: return "unknown status";
  }
}

extern "C" int tv_version(void) { return 100; }
