"""CPU oracle of the ODA decode step (test infrastructure only).

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The product path never does.
"""
from .oda_oracle import *  # noqa: F401,F403
from . import oda_decoder_oracle as decoder  # noqa: F401
from . import oda_train_oracle as train  # noqa: F401
from . import oda_hybrid_oracle as hybrid  # noqa: F401
